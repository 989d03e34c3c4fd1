// Causal forward attention, BF16 inputs, for gfx950 (CDNA4).
//
// What is computed: "ZYFA" README, Usage and Supported configurations
// (causal, GQA head sharing, natural-log LSE, BF16 output, zero padding to
// the query-tile multiple). Query row r sits at position r + delta relative
// to the keys (key c is visible to row r when c <= r + delta): delta = 0
// with seqlen_q == seqlen_k is whole-sequence causal attention; other
// values give the partial results over a range of keys that the README's
// Accuracy note and the RDNA3 page's split-and-merge combine through the
// LSE. Rows that see no key get O = 0 and LSE = -inf.
//
// Structure (one workgroup = 8 waves = 512 threads, persistent):
//  - A job is a pair of query tiles (i, n-1-i) of one (batch, head)
//    (README, Kernel design: work distribution). Each wave owns QG 16-row
//    groups of query rows for the whole key loop: 256-row tiles with two
//    groups, or 128-row tiles with one for shapes with few (batch, head)
//    slices, whose 256-row pairs would leave compute units idle.
//  - Keys stream in 64-key tiles through four-slot K and V rings in LDS,
//    filled by direct global-to-LDS loads (buffer_load ... lds) two tiles
//    (K) and one tile (V) ahead of use; the lag wave group issues the K
//    loads and the lead group the V loads.
//  - Ping-pong (README, Kernel design: ping-pong schedule; the post
//    "Attention at the Power Cap", two wave groups half a tile apart): the
//    two waves that share a SIMD run half a tile apart, so while one issues
//    the matrix instructions of a tile the other computes the softmax of
//    its own; one barrier per interval keeps the groups in step.
//  - Scores are computed transposed, S^T = K Q^T, with K as the MFMA A
//    operand (README, Kernel design: transposed scores), using
//    v_mfma_f32_16x16x32_bf16. Lane (g, n) (g = lane/16, n = lane%16) then
//    holds, for query column n, the keys 16*kb + 4*g + i of each 16-key
//    block kb: a lane owns part of one query row, and P goes from registers
//    straight into the PV product as the B operand.
//  - O^T += V^T P^T with V^T read from LDS by ds_read_b64_tr_b16, which
//    transposes 16-bit values during the read, so the V tile keeps its
//    memory layout in LDS and no transposing pass is needed.
//  - Online softmax in base 2 (log2(e) folded into the scale, one FMA per
//    score before the exponential) with a lazy reference maximum: it moves
//    only when some score passes it by kTau; one wave-wide ballot decides,
//    and the rescale runs out of line (README, Kernel design: lazy
//    rescaling). The causal mask is applied on diagonal tiles only.
//  - Row sums: with LSE requested, an fp32 sum of the unrounded
//    probabilities (so the LSE holds to ~1e-7 relative); otherwise the
//    matrix unit sums the bf16 P (the post "Attention at the Power Cap",
//    row sums on the matrix core with a 2:4 sparse ones operand), so the
//    output is divided by the sum of exactly the rounded weights that
//    multiply V: one v_smfmac_f32_16x16x64_bf16 per 64 keys, whose sparse
//    A operand is all ones with even rows keeping positions {0, 1} and odd
//    rows {2, 3} of every group of four keys, so rows 2r and 2r + 1 of the
//    result add up to the sum over all 64 keys (half the matrix work of
//    two dense 16x16x32 products against ones).
//  - Every conversion rounds to nearest even (README, Kernel design).
#include "device_common.h"
#include "zyfa_internal.h"

namespace zyfa {
namespace {

constexpr int kThreads = 512;
constexpr int kTileK = 64;
constexpr int kSlots = 4;              // K and V ring depth
constexpr float kTau = 8.0f;           // lazy-rescale threshold, log2 units
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRefFloor = -1e30f;      // initial reference maximum, base-2 units

template <int DQK, bool WITH_LSE, int QG>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_bf16_kernel(const AttnArgs a) {
  constexpr int DV = 128;
  constexpr int RW = 16 * QG;                  // query rows per wave (QG 16-row groups)
  constexpr int kTileQ = 8 * RW;               // query rows per tile
  constexpr int KCH = DQK / 8;                 // 16-byte chunks per K row
  constexpr int KPITCH = DQK * 2;              // bytes per K row in LDS
  constexpr int VPITCH = DV * 2;
  constexpr int KSWZ = (KCH % 16 == 0) ? 15 : 7;
  constexpr int K_SLOT = kTileK * KPITCH;
  constexpr int V_SLOT = kTileK * VPITCH;
  constexpr int NC = DQK / 32;                 // MFMA k-steps over d_qk
  constexpr int KLD = K_SLOT / 1024 / 8;       // 1 KiB direct-to-LDS loads per wave per tile
  constexpr int VLD = V_SLOT / 1024 / 8;
  static_assert(KLD * 8 * 1024 == K_SLOT && VLD * 8 * 1024 == V_SLOT, "tile split");
  // LDS fragment prefetch distance of the matrix cluster
  constexpr int kPfV = 4;
  constexpr int kPfK = 4;

  __shared__ __attribute__((aligned(16))) char smem[kSlots * (K_SLOT + V_SLOT)];
  char* const kring = smem;
  char* const vring = smem + kSlots * K_SLOT;
  // the rings' LDS byte addresses, for the direct-to-LDS loads
  const unsigned kring_lds = lds_addr(smem);
  const unsigned vring_lds = kring_lds + kSlots * K_SLOT;

  // work-item and group ids from the hardware registers directly (the
  // device-library accessors are not inlined into a kernel compiled with
  // IEEE mode off, and a call would spill every live register)
  const int tid = (int)__builtin_amdgcn_workitem_id_x();
  const int wg = (int)__builtin_amdgcn_workgroup_id_x();
  const int lane = tid & 63;
  // wave-uniform values live in scalar registers
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int n = lane & 15;
  // Waves w and w + 4 share a SIMD. Waves 4..7 (the lead group, which also
  // holds the query rows with more keys) run half a key tile ahead of waves
  // 0..3 (the lag group).
  const bool lead = wave >= 4;
  // The wave's index within its group, as a scalar: the load addresses
  // built from it then stay in scalar registers (built from the per-lane
  // wave index, each load needs vector address arithmetic and a
  // readfirstlane, and the extra live registers spilled at d_qk = 192).
  const int wq = __builtin_amdgcn_readfirstlane(wave & 3);
  const int ws = __builtin_amdgcn_readfirstlane(wave);
  const int Sq = a.seqlen_q;
  const int Sk = a.seqlen_k;
  const int dl = a.delta;
  const float sl2 = a.scale_log2;
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  // 2:4 sparsity index of the row-sum operand: lane n supplies row n; 2-bit
  // positions of its two values in each of its four groups of four keys,
  // {0, 1} (0b0100) on even rows and {2, 3} (0b1110) on odd rows
  const int sum_idx = (n & 1) ? 0xEEEE : 0x4444;

  for (int it = 0; it < a.jobs_per_wg; ++it) {
    const int2 jv = a.jobs[it * a.num_wgs + wg];
    const int2 job = {__builtin_amdgcn_readfirstlane(jv.x), __builtin_amdgcn_readfirstlane(jv.y)};
    if (job.x < 0) break;
    const int b = job.x / a.nheads;
    const int h = job.x - b * a.nheads;
    const int hk = (int)(((long long)h * a.nheads_k) / a.nheads);

    const char* qbase = (const char*)a.q.ptr + 2 * (b * a.q.stride_b + h * a.q.stride_h);
    const char* kbase = (const char*)a.k.ptr + 2 * (b * a.k.stride_b + hk * a.k.stride_h);
    const char* vbase = (const char*)a.v.ptr + 2 * (b * a.v.stride_b + hk * a.v.stride_h);
    const int qrs = (int)(2 * a.q.stride_s);
    const int krs = (int)(2 * a.k.stride_s);
    const int vrs = (int)(2 * a.v.stride_s);

    // Per-lane byte offsets of the direct-to-LDS tile loads (fixed for the
    // job; the offset of the tile, or of its upper half, goes into the
    // buffer resource, whose extent covers only the rows before seqlen, so
    // later rows read as zeros). One wave group loads each whole tile (the
    // lag group K, the lead group V): wave wq of the group fills
    // instructions I = wq * n + u (n = KLD or VLD) of each 32-row half. Instruction I fills bytes [1024 I, 1024 I + 1024) of the half;
    // lane L's 16 bytes land at p = 1024 I + 16 L, which is row p / pitch,
    // chunk slot (p % pitch) / 16, so the lane fetches the global chunk that
    // belongs in that slot (the same offsets serve both halves, 32 rows
    // apart being a multiple of every swizzle period). K chunks are XOR-swizzled by row so the 16 lanes
    // that read one chunk column of 16 rows hit distinct banks; V chunks are
    // swizzled by even values, keeping the 8-byte halves the transposing
    // read needs intact.
    int kvo[KLD], vvo[VLD];
#pragma unroll
    for (int u = 0; u < KLD; ++u) {
      const int p = (wq * KLD + u) * 1024 + lane * 16;
      const int row = p / KPITCH, x = ((p % KPITCH) >> 4) ^ (row & KSWZ);
      kvo[u] = row * krs + x * 16;
    }
#pragma unroll
    for (int u = 0; u < VLD; ++u) {
      const int p = (wq * VLD + u) * 1024 + lane * 16;
      const int row = p / VPITCH, x = ((p % VPITCH) >> 4) ^ ((row & 7) << 1);
      vvo[u] = row * vrs + x * 16;
    }
    // resource at rows 32 half .. of key tile kt
    auto tile_rsrc = [&](const char* base, int stride, int row_bytes, int kt, int half) {
      const int r0 = kt * kTileK + 32 * half;
      return make_rsrc_words(base + (unsigned long long)r0 * (unsigned)stride,
                             rows_extent(min(Sk - r0, 32), stride, row_bytes));
    };

    const int tA = job.y;
    const int tB = a.n_qtiles - 1 - job.y;
    const int ntiles = (tA == tB) ? 1 : 2;
    for (int tt = 0; tt < ntiles; ++tt) {
      // the longer tile first: the workgroups of one chiplet then stream the
      // same keys at the same time for longer, so K and V stay in its L2
      const int qt = tt == 0 ? tB : tA;
      const int q0 = qt * kTileQ;
      const int qw0 = q0 + wave * RW;
      const int qend = min(q0 + kTileQ, Sq);
      // key tiles that some row of the query tile sees (when any: the
      // tile's last row sees qend + delta keys, capped at seqlen_k)
      const bool any_key = qend + dl > 0;
      const int n_kt = (min(Sk, qend + dl) - 1) / kTileK + 1;
      // this wave's last key tile (the one holding its diagonal), -1 if the
      // wave has no rows or its rows see no key
      const int lk_w = min(Sk - 1, qw0 + RW - 1 + dl);
      const int kt_w = (qw0 < Sq && lk_w >= 0) ? min(lk_w / kTileK, n_kt - 1) : -1;

      // Key tiles are visited in ascending order for the first (longer)
      // query tile of the pair and in descending order for the second. A
      // pair's tiles together span the same number of key tiles for every
      // pair, so the workgroups of a chiplet that have moved on to their
      // second tiles all read the same key tile at the same time and share
      // it in L2. Position j of the visit order is key tile tile_of(j); ring
      // slots follow the position.
      const bool rev = tt == 1;
      auto tile_of = [&](int j) { return rev ? n_kt - 1 - j : j; };
      // whether position j holds a key tile with keys for this wave's rows
      auto has = [&](int j) { return j < n_kt && tile_of(j) <= kt_w; };

      // Q fragments, MFMA B operand: lane (g, n) holds q[row n][32c + 8g .. +7],
      // read through a resource based at the wave's first row.
      const int qr0 = q0 + RW * ws;
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(qbase + (unsigned long long)qr0 * (unsigned)qrs,
                                                  rows_extent(min(Sq - qr0, RW), qrs, 2 * DQK));
      bf16x8 qf[QG][NC];
#pragma unroll
      for (int qg = 0; qg < QG; ++qg)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          qf[qg][c] = __builtin_bit_cast(bf16x8, buf_load16(rq, (16 * qg + n) * qrs + (32 * c + 8 * g) * 2));

      f32x4 o[QG][8];
      f32x4 lacc[QG];
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        lacc[qg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < 8; ++db) o[qg][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // Reference maxima start at a finite floor, so rows that have seen no
      // key yet give exp2(-inf - m) = 0 and rescale factors of 1, never NaN.
      float mref[QG];
      // lazy-rescale threshold in raw score units, (m + tau) / sl2
      float thr[QG];
      float lsum[QG];
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        mref[qg] = kRefFloor;
        thr[qg] = neg_inf();
        lsum[qg] = 0.f;
      }
      // scores of the tile in flight (made by a matrix cluster, turned into
      // P by the next vector cluster) and the bf16 P (made by a vector
      // cluster, multiplied into V by the next matrix cluster)
      f32x4 s[QG][4];
      bf16x8 pb[QG][2];

      auto issue_k = [&](int j) {
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const unsigned base = kring_lds + (j % kSlots) * K_SLOT + hs * (K_SLOT / 2);
          const i32x4 r = tile_rsrc(kbase, krs, 2 * DQK, tile_of(j), hs);
#pragma unroll
          for (int u = 0; u < KLD; ++u) dma16(r, kvo[u], base + (wq * KLD + u) * 1024);
        }
      };
      auto issue_v = [&](int j) {
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const unsigned base = vring_lds + (j % kSlots) * V_SLOT + hs * (V_SLOT / 2);
          const i32x4 r = tile_rsrc(vbase, vrs, 2 * DV, tile_of(j), hs);
#pragma unroll
          for (int u = 0; u < VLD; ++u) dma16(r, vvo[u], base + (wq * VLD + u) * 1024);
        }
      };

      // V^T fragment idx = 8 kc + db (keys 32 kc .., columns 16 db ..), A
      // operand of O^T += V^T P^T: two transposing reads of 4 x 16 blocks.
      auto v_frag = [&](const char* vs, int idx) {
        const int kc = idx >> 3, db = idx & 7;
        u32x2 t[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int row = 32 * kc + 16 * hf + 4 * g + (n >> 2);
          const int x = 2 * db + ((n & 3) >> 1);
          t[hf] = __builtin_bit_cast(u32x2, lds_read_tr16(vs + row * VPITCH + ((x ^ ((row & 7) << 1)) << 4) + (n & 1) * 8));
        }
        return __builtin_bit_cast(bf16x8, u32x4{t[0][0], t[0][1], t[1][0], t[1][1]});
      };
      // K fragment idx = 4 c + kb (key rows 16 kb + n, d 32 c + 8 g ..), A
      // operand of S^T = K Q^T.
      auto k_frag = [&](const char* ks, int idx) {
        const int c = idx >> 2, kb = idx & 3;
        const int row = 16 * kb + n;
        const int x = 4 * c + g;
        return lds_load<bf16x8>(ks + row * KPITCH + ((x ^ (row & KSWZ)) << 4));
      };

      // Matrix cluster at position j: O^T += V^T P^T and the row sum for
      // position j - 1 (P from the previous vector cluster), then the scores
      // S^T = K Q^T at position j.
      auto matrix_cluster = [&](int j) {
        __builtin_amdgcn_s_setprio(1);
        if (j >= 1 && has(j - 1)) {
          const char* vs = vring + ((j - 1) % kSlots) * V_SLOT;
          bf16x8 vfb[kPfV];
#pragma unroll
          for (int u = 0; u < kPfV; ++u) vfb[u] = v_frag(vs, u);
          if (!WITH_LSE) {
#pragma unroll
            for (int qg = 0; qg < QG; ++qg)
              lacc[qg] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(
                  ones, __builtin_shufflevector(pb[qg][0], pb[qg][1], 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15),
                  lacc[qg], sum_idx, 0, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kPfV, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, QG, 0);
          }
#pragma unroll
          for (int idx = 0; idx < 16; ++idx) {
            const bf16x8 cur = vfb[idx % kPfV];
            if (idx + kPfV < 16) vfb[idx % kPfV] = v_frag(vs, idx + kPfV);
#pragma unroll
            for (int qg = 0; qg < QG; ++qg)
              o[qg][idx & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, pb[qg][idx >> 3], o[qg][idx & 7], 0, 0, 0);
            if (idx + kPfV < 16) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, QG, 0);
          }
        }
        if (has(j)) {
          const char* ks = kring + (j % kSlots) * K_SLOT;
          bf16x8 kfb[kPfK];
#pragma unroll
          for (int u = 0; u < kPfK; ++u) kfb[u] = k_frag(ks, u);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kPfK, 0);
#pragma unroll
          for (int idx = 0; idx < 4 * NC; ++idx) {
            const bf16x8 cur = kfb[idx % kPfK];
            if (idx + kPfK < 4 * NC) kfb[idx % kPfK] = k_frag(ks, idx + kPfK);
            const int c = idx >> 2, kb = idx & 3;
#pragma unroll
            for (int qg = 0; qg < QG; ++qg)
              s[qg][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, qf[qg][c], c == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[qg][kb], 0, 0, 0);
            if (idx + kPfK < 4 * NC) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, QG, 0);
          }
        }
        __builtin_amdgcn_s_setprio(0);
      };

      // Vector cluster at position j: causal mask (diagonal tiles), lane
      // maxima, lazy rescale, P = exp2(s * scale - m) rounded to bf16, and
      // the fp32 row sum when the LSE is requested.
      auto vector_cluster = [&](int j) {
        if (!has(j)) return;
        const int kt0 = tile_of(j) * kTileK;
        // ---- causal mask, on diagonal tiles only; score (kb, i) of lane
        // group g is key 16 kb + 4 g + i of the tile. Row r sees keys up to
        // min(r + delta, seqlen_k - 1): the cap masks the zero rows past the
        // last key when every key is visible.
        if (__builtin_expect(kt0 + kTileK - 1 > min(qw0 + dl, Sk - 1), 0)) {
          const float ninf = neg_inf();
#pragma unroll
          for (int qg = 0; qg < QG; ++qg) {
            const int q = min(qw0 + 16 * qg + n + dl, Sk - 1) - kt0 - 4 * g;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i) s[qg][kb][i] = mask_above(s[qg][kb][i], 16 * kb + i, q, ninf);
          }
        }
        // ---- lazy max: lane maxima of the raw scores, one ballot per tile
        float x[QG];
        bool need = false;
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
          float m = fmaxf(fmaxf(s[qg][0][0], s[qg][0][1]), s[qg][0][2]);
#pragma unroll
          for (int e = 3; e < 15; e += 2)
            m = fmaxf(fmaxf(m, s[qg][e >> 2][e & 3]), s[qg][(e + 1) >> 2][(e + 1) & 3]);
          x[qg] = fmaxf(m, s[qg][3][3]);
          need = need || (x[qg] > thr[qg]);
        }
        if (__builtin_expect(wave_any(need), 0)) {
          // Keep this branch real: with f == 1 the multiplies are harmless,
          // so the compiler would otherwise run them on every tile.
          asm volatile("" ::: "memory");
#pragma unroll
          for (int qg = 0; qg < QG; ++qg) {
            const float rm = max_xor32(max_xor16(x[qg])) * sl2;
            const float mn = fmaxf(mref[qg], rm);
            const float f = fast_exp2(mref[qg] - mn);
            lsum[qg] *= f;
            lacc[qg] *= f;
#pragma unroll
            for (int db = 0; db < 8; ++db) o[qg][db] *= f;
            mref[qg] = mn;
            thr[qg] = (mn + kTau) / sl2;
          }
        }
        // ---- P = exp2(s * scale - m), RNE to bf16. Operands are assembled
        // as whole 32-bit words: building them element by element from
        // 16-bit values has been compiled incorrectly (every slot took
        // element 0).
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
          const float nm = -mref[qg];
          float ls = 0.f;
          u32x4 w[2];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            f32x4 p;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              p[i] = fast_exp2(__builtin_fmaf(s[qg][kb][i], sl2, nm));
              if (WITH_LSE) ls += p[i];
            }
            w[kb >> 1][2 * (kb & 1) + 0] = pack_bf16x2(p[0], p[1]);
            w[kb >> 1][2 * (kb & 1) + 1] = pack_bf16x2(p[2], p[3]);
          }
          pb[qg][0] = __builtin_bit_cast(bf16x8, w[0]);
          pb[qg][1] = __builtin_bit_cast(bf16x8, w[1]);
          if (WITH_LSE) lsum[qg] += ls;
        }
      };

      // Ping-pong over intervals closed by one barrier each. In interval i
      // the lead group runs the vector cluster of position i - 1 and then
      // the matrix cluster of position i; the lag group runs the matrix
      // cluster of position i - 1 and then its vector cluster. On every SIMD
      // one wave is in a matrix cluster while the other computes a softmax.
      // Interval i reads K(i - 1), K(i), V(i - 2) and V(i - 1). The lag
      // group issues K(i + 2) between its two clusters and the lead group
      // issues V(i + 1) at the start of the interval, each into the slots
      // last read in interval i - 1 (four-slot rings); before the barrier
      // each wave waits for the loads it issued one interval earlier (read
      // from interval i + 1 on). A wave that issues direct-to-LDS loads is
      // held until the address unit has accepted them, so the loads are
      // split where each group has slack: issued by one group alone, they
      // lengthen that group's chain past the other's. The last position
      // with work for the lag group is n_kt - 1 in descending order and its
      // last key tile in ascending order; its PV runs two intervals later. A
      // query tile whose rows see no key skips the loop.
      const int lag_last = rev ? n_kt - 1 : (q0 + 4 * RW - 1 + dl >= 0 ? min((q0 + 4 * RW - 1 + dl) / kTileK, n_kt - 1) : -1);
      const int n_int = max(n_kt + 1, lag_last + 3);
      __syncthreads();   // the previous query tile's last reads of the rings are done
      if (any_key) {
        if (lead) {
          issue_v(0);
        } else {
          issue_k(0);
          if (n_kt > 1) issue_k(1);
        }
        wait_vm<0>();
        __syncthreads();
        for (int i = 0; i < n_int; ++i) {
          if (lead) {
            if (i + 1 < n_kt) issue_v(i + 1);
            if (i >= 1) vector_cluster(i - 1);
            matrix_cluster(i);
            if (i + 1 < n_kt) wait_vm<2 * VLD>();
            else wait_vm<0>();
          } else {
            if (i >= 1) matrix_cluster(i - 1);
            if (i + 2 < n_kt) issue_k(i + 2);
            if (i >= 1) vector_cluster(i - 1);
            if (i + 2 < n_kt) wait_vm<2 * KLD>();
            else wait_vm<0>();
          }
          __syncthreads();
        }
      }

      // ---- epilogue: O / l (RNE to bf16), LSE = ln2 * (m + log2 l); rows
      // that saw no key (l = 0) get O = 0 and LSE = -inf
      if (qw0 < Sq) {
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
          float lt;
          if (WITH_LSE) {
            lt = lsum[qg] + swap16(lsum[qg]);
            lt += __shfl_xor(lt, 32);
          } else {
            lt = lacc[qg][0] + lacc[qg][1];   // an even and an odd row of the sparse sum
          }
          const float inv = lt > 0.f ? 1.0f / lt : 0.f;
          const int q = qw0 + 16 * qg + n;
          if (q < Sq) {
            __bf16* orow = (__bf16*)a.out + (b * a.o_stride_b + h * a.o_stride_h + (long long)q * a.o_stride_s);
#pragma unroll
            for (int db = 0; db < 8; ++db) {
              const u32x2 w = {pack_bf16x2(o[qg][db][0] * inv, o[qg][db][1] * inv),
                               pack_bf16x2(o[qg][db][2] * inv, o[qg][db][3] * inv)};
              *reinterpret_cast<u32x2*>(orow + 16 * db + 4 * g) = w;
            }
            if (WITH_LSE && g == 0)
              a.lse[((long long)b * a.nheads + h) * Sq + q] = (mref[qg] + fast_log2(lt)) * kLn2;
          }
        }
      }
    }
  }
}

}  // namespace

template <int DQK, int QG>
static void launch_bf16(const AttnArgs& a, bool with_lse, dim3 gd, dim3 bd, hipStream_t s) {
  if (with_lse) hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, true, QG>), gd, bd, 0, s, a);
  else hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, false, QG>), gd, bd, 0, s, a);
}

hipError_t launch_attn_bf16(const AttnArgs& a, int d_qk, bool with_lse, int tile_q, int grid, hipStream_t s) {
  const dim3 gd(grid), bd(kThreads);
  if (tile_q != 128 && tile_q != 256) return hipErrorInvalidValue;
  const bool tall = tile_q == 256;
  if (d_qk == 128) {
    if (tall) launch_bf16<128, 2>(a, with_lse, gd, bd, s);
    else launch_bf16<128, 1>(a, with_lse, gd, bd, s);
  } else {
    if (tall) launch_bf16<192, 2>(a, with_lse, gd, bd, s);
    else launch_bf16<192, 1>(a, with_lse, gd, bd, s);
  }
  return hipGetLastError();
}

}  // namespace zyfa

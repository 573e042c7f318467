// Sparse gather attention over selected latent rows (gfx950).
//
// What it computes ("IndexShare", LLM Architecture Gallery, section "Why The
// Indexer Becomes Expensive": the main attention runs only over the selected
// subset; "GLM-5.2 and IndexShare for Long-Context Sparse Attention", section
// "What IndexShare reuses": every layer, shared or not, computes its own
// attention weights and value combinations over the shared positions):
//     o[t,h,:] = sum_j softmax_j(sm_scale * q[t,h,:] . kv[idx_j,:]) * kv[idx_j, :Dv]
// over the slots j of row t whose idx lies in [0, kv_len).  The latent row is
// the key; its first Dv dims are the value.
//
// Layout of the work
//   * one wave = one (query row, slot range); all Hq <= 16 heads of the row
//     share every gathered latent row, so each gathered byte feeds 16 heads;
//   * 16 slots per step.  The step's 16 latent rows are gathered with
//     coalesced loads: one instruction moves 1 KB of one row (consecutive
//     lanes, consecutive 16-byte pieces, the row id uniform), so the vector L1
//     sees one tag lookup per cache line instead of one per lane (with the
//     pieces spread the way the MFMA operand wants them, 16 rows per
//     instruction, the L1's tag rate bounded the kernel).  Two named register
//     buffers alternate, so the next step's rows are in flight while this
//     step computes, and index words are loaded two steps ahead.  The
//     buffers and the query slice are held in AGPRs (MFMA operands and LDS
//     stores may come from either register file), the output accumulators
//     and the LDS operand reads in VGPRs;
//   * each step parks its rows in a wave-private LDS tile (one 16-byte store
//     per register) whose row stride is 8 or 40 (mod 64) dwords, so the
//     transposed value reads and the key-operand reads below are
//     bank-conflict free.  (Direct HBM -> LDS loads of the same tile measured
//     about 40% slower than this register path at L = 128K.)
//   * S^T = KV . Q^T with v_mfma_f32_16x16x32_bf16 (M = keys, N = heads, the
//     query slice stays in registers; the key operand is read from the tile
//     several MFMAs ahead of its use), so lane l ends with 4 logits of head
//     l%16 -- exactly the B-operand layout of the P.V product below;
//   * the value part of the 16 rows is read straight from the tile by
//     ds_read_b64_tr_b16 (lane (dv, key group) gets 4 keys of one value dim)
//     as the A operand of O^T = V^T . P^T (v_mfma_f32_16x16x16_bf16), also
//     read ahead of use.  (Without the read-ahead every MFMA waited for its
//     own LDS read: about 4,000 cycles per step against about 550 of MFMA
//     work.  A second tile per wave, with two steps of gathers in flight,
//     measured no faster, and neither did four waves per row.)
//   * online softmax in base 2 against a reference max that may trail the
//     running max by up to 2^8, so the accumulators are rescaled only when a
//     head's max jumps further (rarely);
//   * few rows (decode): the four waves of a workgroup share one (row, split),
//     each taking a quarter of its slots, and merge their (o, m, l) through
//     LDS; with several splits per row the merged partials go to the
//     workspace and a merge kernel combines them, or, for a layer followed by
//     another such launch in a layer group, that launch's prologue does.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ix {

namespace {

constexpr int kWavesPerWG = 4;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kSlack = 8.0f;   // how far the softmax reference may trail the max (log2 units)

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t* lds_v4s_ptr;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Wave-private tile of one 16-slot step, generic layout: row r (D bf16 = C
// 16-byte pieces) at byte r * RS, RS = 16 * CP with CP the smallest piece
// count >= C that is 2 (mod 8) pieces, i.e. 8 or 40 (mod 64) dwords: the 8
// rows x 32 bytes a half-wave of a transposed value read touches then fall in
// 8 disjoint bank groups.  Lane l of gather load j fetches slot s = 64 j + l,
// i.e. row s / CP, piece s % CP, and parks it at byte 16 s; pad pieces and the
// slack of the last load repeat a valid piece of the same or the last row.
template <int KS>
struct GTile {
  static constexpr bool kLatent = false;
  static constexpr int D = 32 * KS;
  static constexpr int C = D / 8;
  static constexpr int CP = C + ((2 - C % 8) + 8) % 8;
  static constexpr int RS = 16 * CP;
  static constexpr int NI = (16 * CP + kWave - 1) / kWave;   // gather loads per step
  static constexpr int bytes = NI * kWave * 16;
  static constexpr int RPI = (kWave + CP - 1) / CP + 1;       // rows one load can touch
  static_assert(CP % 8 == 2, "row stride 2 (mod 8) pieces");
  // byte offset of the key operand (row n16, k-group g of k-step ks) and of
  // a row's value part
  __device__ static __forceinline__ int qk_off(int n16, int ks, int g) { return n16 * RS + 64 * ks + 16 * g; }
  __device__ static __forceinline__ int v_off(int row) { return row * RS; }
};

// The 576-wide latent row (V = its first 512 dims = 1 KB): one gather load
// per row moves the value part (64 lanes x 16 bytes, the row id uniform over
// the load, so its address is a scalar base plus a lane constant), parked in
// a value region of stride 1056 bytes (8 (mod 64) dwords, as above); two loads
// move the 16 rows' 128-byte rope parts (8 lanes per row), parked in a rope
// region of stride 144 bytes (36 (mod 64) dwords: the 8 rows one 16-byte
// operand read phase touches fall in disjoint bank groups).
struct GTileLatent {
  static constexpr bool kLatent = true;
  static constexpr int D = 576, Dv = 512;
  static constexpr int RSV = 1056;
  static constexpr int ROPE = 16 * RSV;
  static constexpr int RSR = 144;
  static constexpr int NR = 2;                                  // rope loads (8 rows each)
  static constexpr int NI = 16 + NR;                            // gather loads per step
  static constexpr int bytes = ROPE + 16 * RSR;
  __device__ static __forceinline__ int qk_off(int n16, int ks, int g) {
    return ks < 16 ? n16 * RSV + 64 * ks + 16 * g : ROPE + n16 * RSR + 64 * (ks - 16) + 16 * g;
  }
  __device__ static __forceinline__ int v_off(int row) { return row * RSV; }
};

// LDS operand reads issued ahead of their MFMAs, and the instruction classes
// of the scheduling-group hints that place them (AMDGPU sched_group_barrier
// masks)
constexpr int kQkAhead = 6, kPvAhead = 8;
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;

template <int KS, int MT>
struct TileOf {
  using type = GTile<KS>;
};
template <>
struct TileOf<18, 32> {
  using type = GTileLatent;
};

// LDS of a workgroup: one tile per wave; after the slot loop the tiles are
// reused as the buffer of the in-workgroup merge (two waves' accumulators),
// then the merge's per-wave (m, l) of every head.
template <int KS, int MT>
struct AttnLds {
  static constexpr int wave_bytes = (TileOf<KS, MT>::type::bytes + 15) / 16 * 16;
  static constexpr int tiles = kWavesPerWG * wave_bytes;
  static constexpr int merge = 2 * MT * kWave * 16;
  static constexpr int stat_off = ((tiles > merge ? tiles : merge) + 15) / 16 * 16;
  static constexpr int comb_off = stat_off + 2 * kWavesPerWG * 16 * 4;   // fused merge: [2][64] weights, [2][2] stats
  static constexpr int bytes = comb_off + (2 * 64 + 4) * 4;
  static_assert(bytes <= 160 * 1024, "LDS of one workgroup");
};

// Merge of split partials, per item (row, head): base-2 log-sum-exp weights
// exp2(m_s - M) / L of the splits from one wave, then each of 128 threads
// folds 4 consecutive value dims (Dv <= 512) over the splits in ascending
// split order.  Used by the merge kernel and, for a launch chained behind
// another, in the later launch's prologue; the same code gives both the same
// bits.  The first kMergePre splits' partials are loaded before the weights
// are known (split indices clamped to the last split; the weights of slots
// past it are never used).
constexpr int kMergePre = 8;

__device__ __forceinline__ void merge_load(const CombineArgs& c, int item, int dv, f32x4 (&v)[kMergePre]) {
  const int r = item / c.Hq, h = item % c.Hq;
  const float* po = c.part_o + ((int64_t)r * c.splits * 16 + h) * c.Dv + min(dv, c.Dv - 4);
#pragma unroll
  for (int u = 0; u < kMergePre; ++u)
    v[u] = *reinterpret_cast<const f32x4*>(po + (int64_t)min(u, c.splits - 1) * 16 * c.Dv);
}

// Lane s of the weight wave: split min(s, S-1)'s (m, l) (the lanes past the
// last split are masked where the weights are formed, not here, so nothing
// waits for these loads before it has to).
__device__ __forceinline__ void merge_ml_load(const CombineArgs& c, int item, int lane, float& ms, float& ls) {
  const int r = item / c.Hq, h = item % c.Hq;
  const float* ml = c.part_ml + ((int64_t)r * c.splits * 16 + h) * 2;   // split s at + s*32
  const int sl = min(lane, c.splits - 1);
  ms = ml[(int64_t)sl * 32];
  ls = ml[(int64_t)sl * 32 + 1];
}

// One whole wave: wgt[s] for s < S and stat = (M, L).
__device__ __forceinline__ void merge_weights(float ms_raw, float ls_raw, int lane, int S, float* wgt, float* stat) {
  const float ms = lane < S ? ms_raw : -INFINITY;
  const float ls = lane < S ? ls_raw : 0.0f;
  float M = ms;
#pragma unroll
  for (int dd = 32; dd >= 1; dd >>= 1) M = fmaxf(M, __shfl_xor(M, dd));
  const float e = (ms == -INFINITY) ? 0.0f : exp2f(ms - M);
  float L = ls * e;
#pragma unroll
  for (int dd = 32; dd >= 1; dd >>= 1) L += __shfl_xor(L, dd);
  if (lane < S) wgt[lane] = L > 0.0f ? e / L : 0.0f;
  if (lane == 0) {
    stat[0] = M;
    stat[1] = L;
  }
}

__device__ __forceinline__ void merge_fold(const CombineArgs& c, int item, int dv, const f32x4 (&v)[kMergePre],
                                           const float* wgt, const float* stat) {
  const int r = item / c.Hq, h = item % c.Hq;
  const int S = c.splits;
  if (dv < c.Dv) {
    f32x4 acc = f32x4{};
#pragma unroll
    for (int u = 0; u < kMergePre; ++u)
      if (u < S) acc += v[u] * wgt[u];
    const float* po = c.part_o + ((int64_t)r * S * 16 + h) * c.Dv + dv;
    for (int sp = kMergePre; sp < S; ++sp) acc += *reinterpret_cast<const f32x4*>(po + (int64_t)sp * 16 * c.Dv) * wgt[sp];
    const u32x2 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    *reinterpret_cast<u32x2*>(c.out + ((int64_t)r * c.Hq + h) * c.Dv + dv) = o;
  }
  if (dv == 0 && c.lse)
    c.lse[(int64_t)r * c.Hq + h] = stat[1] > 0.0f ? (stat[0] + log2f(stat[1])) * kLn2 : -INFINITY;
}

// Workgroup barrier that orders LDS only (s_barrier after this wave's LDS
// operations), so loads in flight are not drained.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int KS, int MT, int WPI>
__global__ __launch_bounds__(kWavesPerWG * kWave, 1) void sparse_attn_kernel(AttnArgs a) {
  constexpr int D = 32 * KS, Dv = 16 * MT;
  using G = typename TileOf<KS, MT>::type;
  using L = AttnLds<KS, MT>;
  static_assert(WPI == 1 || WPI == kWavesPerWG, "a (row, split) has one wave or the whole workgroup");
  extern __shared__ __align__(16) unsigned char smem[];
  // the wave index is uniform across the wave; saying so keeps the slot
  // range scalar and the loop exits uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  const int n16 = l & 15, g = l >> 4;
  const int item = WPI == 1 ? blockIdx.x * kWavesPerWG + wave : blockIdx.x;
  if (item >= a.rows * a.splits) return;     // whole workgroup when WPI > 1
  const int r = item / a.splits, sp = item % a.splits;
  const int b = r / a.n_q;
  unsigned char* const tile = smem + wave * L::wave_bytes;

  // An earlier launch's partials merged here (whole workgroups, two items per
  // pass, 128 threads each): the first pass's partials and split statistics
  // are loaded ahead of everything else (every lane loads, no branch), so
  // waiting for them waits for nothing of this launch; the merge itself runs
  // once this launch's index words are requested, before its query slice and
  // gathers (merging while the first gathers were in flight measured slower).
  const CombineArgs mc = a.prev;          // by value (a reference into the kernel arguments costs a stack frame)
  const int m_items = WPI > 1 && mc.splits > 1 ? mc.rows * mc.Hq : 0;
  const int m_half = threadIdx.x >> 7, m_tid = threadIdx.x & 127;
  f32x4 mv[kMergePre];
  float m_ms = -INFINITY, m_ls = 0.0f;
  if (m_items > 0) {
    const int it0 = min(2 * (int)blockIdx.x + m_half, m_items - 1);
    merge_load(mc, it0, 4 * m_tid, mv);
    merge_ml_load(mc, it0, m_tid & (kWave - 1), m_ms, m_ls);
  }
  __builtin_amdgcn_sched_barrier(0);

  // Query slice as the B operand: head n16, elements [32ks + 8g, +8) -- the
  // MFMA's k-group g of step ks; the key operand is read the same way.
  // Lanes of heads past Hq load head 0's query (in bounds, finite): their
  // logits and outputs are never stored.  The loads are unconditional, so no
  // branch splits them.
  const bool hq_ok = n16 < a.Hq;
  bf16x8 qf[KS];

  int j0 = sp * a.slots_per_split;
  int j1 = min(a.k, j0 + a.slots_per_split);
  if (WPI > 1) {                              // this wave's quarter of the split
    const int per = a.slots_per_split / WPI;
    j0 = min(j1, j0 + wave * per);
    j1 = min(j1, j0 + per);
  }
  const int32_t* irow = a.idx + (int64_t)r * a.k;
  const uint16_t* kvb = a.kv + (int64_t)b * a.kv_bstride;

  f32x4 oacc[MT];                         // zeroed after a chained merge (not live beside it)
  float m_run = -INFINITY, l_run = 0.0f;

  // Loads are unconditional: exec-masked load branches make the compiler's
  // memory-counter waits fall back to draining every load in flight, which
  // would stall each step on the next step's prefetch.  An index word past
  // the range reads an in-row slot and becomes -1; an invalid slot gathers
  // row 0, whose logit is masked to -inf and whose value row is weighted by 0.
  // Lane n16 (every g) loads the index word of slot c0 + n16; the word is
  // checked only when its step is gathered (a check right after the load
  // would wait for it, and loads complete in order, so for every gather
  // issued before it).
  auto slot_word = [&](int c0) -> int { return irow[min(c0 + n16, a.k - 1)]; };
  // The 16 latent rows of the step at slot c0 (index word rid) into register
  // buffer kf; returns whether this lane's slot (n16) is valid.
  auto fetch = [&](int c0, int rid, bf16x8 (&kf)[G::NI]) -> bool {
    const bool valid = c0 + n16 < j1 && rid >= 0 && (int64_t)rid < a.kv_len;
    const int rid_c = valid ? rid : 0;
    int rs[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) rs[q] = __builtin_amdgcn_readlane(rid_c, q);
    if constexpr (G::kLatent) {
#pragma unroll
      for (int q = 0; q < 16; ++q) kf[q] = *reinterpret_cast<const bf16x8*>(kvb + (int64_t)rs[q] * D + 8 * l);
#pragma unroll
      for (int h = 0; h < G::NR; ++h) {
        const int rid_h = __shfl(rid_c, 8 * h + (l >> 3));
        kf[16 + h] = *reinterpret_cast<const bf16x8*>(kvb + (int64_t)rid_h * D + G::Dv + 8 * (l & 7));
      }
    } else {
#pragma unroll
      for (int j = 0; j < G::NI; ++j) {
        const int sl = kWave * j + l;
        const int row = sl / G::CP;                 // >= 16 only in the last load's slack
        const int pc = min(sl - row * G::CP, G::C - 1);
        const int r0 = (kWave * j) / G::CP;         // constant once the loop is unrolled
        int rq = rs[min(r0, 15)];
#pragma unroll
        for (int dr = 1; dr < G::RPI; ++dr)
          if (row == r0 + dr) rq = rs[min(r0 + dr, 15)];
        kf[j] = *reinterpret_cast<const bf16x8*>(kvb + (int64_t)rq * D + 8 * pc);
      }
    }
    return valid;
  };

  // Park a step's gathered rows kf in the tile (nothing when no slot is
  // valid); returns the valid-slot mask (bit n: slot n, from lanes 0..15).
  // The stores follow the last reads of that tile in program order, and a
  // wave's LDS operations complete in order.
  auto park = [&](bf16x8 (&kf)[G::NI], bool valid, unsigned char* tile) -> uint32_t {
    // Register-class hint: the buffers live in AGPRs (the loads write them
    // there, the stores read them there), leaving the VGPRs to the output
    // accumulators and the read-ahead of the LDS operands.  The empty asm
    // reads the gathered values, which the stores below wait for anyway.
#pragma unroll
    for (int j = 0; j < G::NI; ++j) asm volatile("" : "+a"(kf[j]));
    const uint32_t vm = (uint32_t)__ballot(valid) & 0xFFFFu;
    if (vm == 0u) return 0u;
    if constexpr (G::kLatent) {
#pragma unroll
      for (int q = 0; q < 16; ++q) *reinterpret_cast<bf16x8*>(tile + G::v_off(q) + 16 * l) = kf[q];
#pragma unroll
      for (int h = 0; h < G::NR; ++h)
        *reinterpret_cast<bf16x8*>(tile + G::ROPE + (8 * h + (l >> 3)) * G::RSR + 16 * (l & 7)) = kf[16 + h];
    } else {
#pragma unroll
      for (int j = 0; j < G::NI; ++j) *reinterpret_cast<bf16x8*>(tile + 16 * (kWave * j + l)) = kf[j];
    }
    // the stores are visible to this wave's later LDS reads; the compiler
    // must not move reads of other lanes' pieces above them
    asm volatile("" ::: "memory");
    return vm;
  };

  // One 16-slot step on a parked tile: S^T = KV . Q^T, online softmax,
  // O^T += V^T . P^T.
  auto step = [&](uint32_t vm, const unsigned char* tile) {
    if (vm == 0u) return;
    // one accumulator chain, so the MFMAs consume the key operand reads in
    // the order they are issued (LDS reads complete in order; a chain taken
    // out of that order waits for every earlier read); the reads run
    // kQkAhead MFMAs ahead of their use (left alone, the compiler waits for
    // each read right before its MFMA)
    f32x4 sacc = f32x4{};
    {
      constexpr int A = KS < kQkAhead ? KS : kQkAhead;
      bf16x8 kk[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kk[ks] = *reinterpret_cast<const bf16x8*>(tile + G::qk_off(n16, ks, g));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk[ks], qf[ks], sacc, 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, A, 0);
#pragma unroll
      for (int i = 0; i < KS - A; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, A, 0);
    }
    float z[4];
    float cmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = ((vm >> (4 * g + i)) & 1u) ? sacc[i] * a.scale_log2 : -INFINITY;
      cmax = fmaxf(cmax, z[i]);
    }
    const auto fmax_op = [](float x, float y) { return fmaxf(x, y); };
    const auto add_op = [](float x, float y) { return x + y; };
    cmax = xor32_op(xor16_op(cmax, fmax_op), fmax_op);
    // The reference m_run may trail the running max by up to kSlack (log2
    // units): every p = 2^(z - m_run) then stays below 2^kSlack, far inside
    // the fp32 and bf16 ranges, and the normalised softmax does not depend on
    // the reference.  The accumulators are rescaled only when a head's max
    // jumps further, which after the first step is rare.
    const bool jump = cmax > m_run + kSlack;     // always true on a head's first valid step
    if (__builtin_expect(__ballot(jump) != 0, 0)) {
      const float m_new = jump ? cmax : m_run;
      const float alpha = jump ? exp2f(m_run - m_new) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) oacc[mt] *= alpha;
      m_run = m_new;
    }
    float pv[4];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = m_run == -INFINITY ? 0.0f : exp2f(z[i] - m_run);
      psum += pv[i];
    }
    psum = xor32_op(xor16_op(psum, add_op), add_op);
    l_run += psum;
    const uint32_t p01 = pack_bf16x2(pv[0], pv[1]), p23 = pack_bf16x2(pv[2], pv[3]);
    const i16x4 pb = __builtin_bit_cast(i16x4, u32x2{p01, p23});
    // transposed read: lane (n16, g) supplies 4 value dims of key 4g + n16/4
    // and receives value dim 16mt + n16 of keys 4g .. 4g+3
    const uint16_t* vrow = reinterpret_cast<const uint16_t*>(tile + G::v_off(4 * g + (n16 >> 2))) + 4 * (n16 & 3);
    // the value reads run kPvAhead MFMAs ahead of their use
    {
      constexpr int A = MT < kPvAhead ? MT : kPvAhead;
      v4s_t vt[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) vt[mt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(vrow + 16 * mt));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        oacc[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, vt[mt]), pb, oacc[mt], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, A, 1);
#pragma unroll
      for (int i = 0; i < MT - A; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 1);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, A, 1);
    }
    // the next step's stores come after these reads (in-order LDS); keep
    // the compiler from moving them above
    asm volatile("" ::: "memory");
  };

  // Two named buffers in turn (unrolled by 2): the step on one runs while the
  // other's gathers are in flight; a step's rows are parked right after the
  // previous step's compute is issued, so the stores overlap its P.V MFMAs.
  // A loop-carried copy of the buffer would make the compiler wait for those
  // gathers at every step.
  // The first two steps' gathers are issued together, so the second does not
  // wait for the first to land (a decode wave walks only a few steps).
  bf16x8 kA[G::NI], kB[G::NI];
  const int w0 = slot_word(j0), w1 = slot_word(j0 + 16);
  int r1 = slot_word(j0 + 32), r2 = slot_word(j0 + 48);
  if (m_items > 0) {                     // the earlier launch's merge
    float* mw = reinterpret_cast<float*>(smem + L::comb_off);     // [2][64] weights, then [2][2] stats
    for (int base = 2 * (int)blockIdx.x; base < m_items; base += 2 * (int)gridDim.x) {
      const int it = base + m_half;
      const bool ok = it < m_items;
      if (base != 2 * (int)blockIdx.x) {     // a later pass: the previous one's weights were read
        lds_barrier();
        const int itc = min(it, m_items - 1);
        merge_load(mc, itc, 4 * m_tid, mv);
        merge_ml_load(mc, itc, m_tid & (kWave - 1), m_ms, m_ls);
      }
      if (ok && m_tid < kWave) merge_weights(m_ms, m_ls, m_tid, mc.splits, mw + 64 * m_half, mw + 128 + 2 * m_half);
      lds_barrier();
      if (ok) merge_fold(mc, it, 4 * m_tid, mv, mw + 64 * m_half, mw + 128 + 2 * m_half);
    }
  }
  {
    const uint16_t* qrow = a.q + ((int64_t)r * a.Hq + (hq_ok ? n16 : 0)) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
  }
  bool vA = fetch(j0, w0, kA);
  bool vB = fetch(j0 + 16, w1, kB);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) oacc[mt] = f32x4{};

  if (j0 < j1) {
    uint32_t vm = park(kA, vA, tile);
    // Register-class hint: the query slice stays in AGPRs (an MFMA operand may
    // come from either file).  The empty asm reads it, so it sits after the
    // first park, which has waited for every earlier load anyway; placed at the
    // query loads it held the index words and the first gathers behind them.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+a"(qf[ks]));
    for (int c0 = j0;; c0 += 32) {
      // tile: step c0; kB: step c0+16 in flight; r1, r2: index words of c0+32, c0+48
      step(vm, tile);
      if (c0 + 16 >= j1) break;
      vm = park(kB, vB, tile);
      vA = fetch(c0 + 32, r1, kA);
      r1 = r2;
      r2 = slot_word(c0 + 64);
      step(vm, tile);
      if (c0 + 32 >= j1) break;
      vm = park(kA, vA, tile);
      vB = fetch(c0 + 48, r1, kB);
      r1 = r2;
      r2 = slot_word(c0 + 80);
    }
  }

  // oacc[mt][i] = O^T[dv = 16mt + 4g + i][head n16]
  if constexpr (WPI > 1) {
    // merge the waves: common max per head, rescale, then sum the
    // accumulators pairwise through LDS (waves 2,3 -> 0,1, then 1 -> 0)
    float* st_m = reinterpret_cast<float*>(smem + L::stat_off);
    float* st_l = st_m + kWavesPerWG * 16;
    f32x4* buf = reinterpret_cast<f32x4*>(smem);
    __syncthreads();                          // every wave is done with its tile
    if (g == 0) {
      st_m[wave * 16 + n16] = m_run;
      st_l[wave * 16 + n16] = l_run;
    }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWavesPerWG; ++w) M = fmaxf(M, st_m[w * 16 + n16]);
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < kWavesPerWG; ++w) {
      const float mw = st_m[w * 16 + n16];
      L += mw == -INFINITY ? 0.0f : st_l[w * 16 + n16] * exp2f(mw - M);
    }
    const float sc = m_run == -INFINITY ? 0.0f : exp2f(m_run - M);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oacc[mt] *= sc;
    if (wave >= 2)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) buf[((wave - 2) * MT + mt) * kWave + l] = oacc[mt];
    __syncthreads();
    if (wave < 2)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) oacc[mt] += buf[(wave * MT + mt) * kWave + l];
    __syncthreads();
    if (wave == 1)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) buf[mt * kWave + l] = oacc[mt];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oacc[mt] += buf[mt * kWave + l];
    m_run = M;
    l_run = L;
  }
  if (a.splits == 1) {
    if (hq_ok) {
      const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
      uint16_t* orow = a.out + ((int64_t)r * a.Hq + n16) * Dv + 4 * g;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x2 v = {pack_bf16x2(oacc[mt][0] * inv, oacc[mt][1] * inv),
                         pack_bf16x2(oacc[mt][2] * inv, oacc[mt][3] * inv)};
        *reinterpret_cast<u32x2*>(orow + 16 * mt) = v;
      }
      if (a.lse && g == 0)
        a.lse[(int64_t)r * a.Hq + n16] = l_run > 0.0f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    }
  } else {
    const int64_t pi = ((int64_t)r * a.splits + sp) * 16 + n16;
    float* po = a.part_o + pi * Dv + 4 * g;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<f32x4*>(po + 16 * mt) = oacc[mt];
    if (g == 0) {
      a.part_ml[pi * 2] = m_run;
      a.part_ml[pi * 2 + 1] = l_run;
    }
  }
}

// Merge of one item (row, head) of a launch's split partials per workgroup.
__global__ __launch_bounds__(128) void attn_combine_kernel(CombineArgs c) {
  __shared__ float wgt[64];
  __shared__ float stat[2];
  const int item = blockIdx.x;              // r * Hq + h
  const int dv = threadIdx.x * 4;
  f32x4 v[kMergePre];
  merge_load(c, item, dv, v);
  if (threadIdx.x < kWave) {
    float ms, ls;
    merge_ml_load(c, item, threadIdx.x, ms, ls);
    merge_weights(ms, ls, threadIdx.x, c.splits, wgt, stat);
  }
  __syncthreads();
  merge_fold(c, item, dv, v, wgt, stat);
}

template <int KS, int MT, int WPI>
hipError_t launch_attn_w(const AttnArgs& a, hipStream_t s) {
  const size_t lds = (size_t)AttnLds<KS, MT>::bytes;
  const void* fn = reinterpret_cast<const void*>(&sparse_attn_kernel<KS, MT, WPI>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t items = (int64_t)a.rows * a.splits;
  dim3 grid((unsigned)(WPI == 1 ? (items + kWavesPerWG - 1) / kWavesPerWG : items));
  hipLaunchKernelGGL((sparse_attn_kernel<KS, MT, WPI>), grid, dim3(kWavesPerWG * kWave), lds, s, a);
  return hipGetLastError();
}

template <int KS, int MT>
hipError_t launch_attn_t(const AttnArgs& a, hipStream_t s, bool defer_combine) {
  if (a.wpi != 1 && a.wpi != kWavesPerWG) return hipErrorInvalidValue;
  if (a.wpi > 1 && a.slots_per_split % (16 * kWavesPerWG) != 0) return hipErrorInvalidValue;
  if (a.prev.splits > 1 && (a.wpi == 1 || a.prev.Dv > 512 || a.prev.Dv % 4 != 0 || a.prev.Hq > 16 ||
                            a.prev.splits > 64))
    return hipErrorInvalidValue;
  hipError_t e = a.wpi == 1 ? launch_attn_w<KS, MT, 1>(a, s) : launch_attn_w<KS, MT, kWavesPerWG>(a, s);
  if (e != hipSuccess || a.splits == 1 || defer_combine) return e;
  return launch_attn_combine(CombineArgs{a.part_o, a.part_ml, a.out, a.lse, a.rows, a.Hq, a.splits, 16 * MT}, s);
}

}  // namespace

bool attn_shape_supported(int d_qk, int d_v) {
  return (d_qk == 576 && d_v == 512) || (d_qk == 128 && (d_v == 96 || d_v == 128)) ||
         (d_qk == 64 && d_v == 64);
}

hipError_t launch_sparse_attn(const AttnArgs& a, int d_qk, int d_v, hipStream_t s, bool defer_combine) {
  if (d_qk == 576 && d_v == 512) return launch_attn_t<18, 32>(a, s, defer_combine);
  if (d_qk == 128 && d_v == 96) return launch_attn_t<4, 6>(a, s, defer_combine);
  if (d_qk == 128 && d_v == 128) return launch_attn_t<4, 8>(a, s, defer_combine);
  if (d_qk == 64 && d_v == 64) return launch_attn_t<2, 4>(a, s, defer_combine);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_combine(const CombineArgs& c, hipStream_t s) {
  if (c.splits <= 1) return hipSuccess;
  if (c.Dv > 512 || c.Dv % 4 != 0 || c.Hq > 16 || c.splits > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(c.rows * c.Hq)), dim3(128), 0, s, c);
  return hipGetLastError();
}

}  // namespace ix

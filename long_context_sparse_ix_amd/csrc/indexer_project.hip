// Indexer inputs from hidden states (gfx950).
//
// What it computes ("IndexCache: Killing the Indexer's O(NL^2) Bottleneck"
// notes, section 1: the indexer is a small low-rank module with few heads;
// the shapes are this library's reading): one bf16 row x [d_in] per query
// and one bf16 weight W [N = H*d + H][d_in] give
//     y = x . W^T,  q_I = bf16(y[0, H*d))  (nearest, ties to even),
//                   w   = y[H*d, N)        (fp32)
// as one GEMM with fp32 accumulation on bf16 MFMA and a split epilogue.
//
// Layout of the work
//   * a workgroup of 4 waves computes a BM x BN output tile, each wave a
//     (BM/2) x (BN/2) quarter as blocks of v_mfma_f32_32x32x16_bf16, stepping
//     K by 64; 256 x 256 tiles (a 256-register accumulator per wave, in AGPRs)
//     when there are rows enough to fill the chip, 64 x 64 tiles for a few
//     rows (decode batches), where the 256-row tiles would mostly multiply
//     padding on a few CUs;
//   * x and W tiles go HBM -> LDS with direct buffer loads (16 bytes a lane,
//     one 1 KB instruction per 8 rows of 128 bytes) into a ring of STAGES LDS
//     stages; one barrier per step, after which step kt + STAGES is loaded
//     into the stage step kt has finished with;
//   * each step is four phases of 16 k: a phase reads the next slice's
//     fragments (in the order its MFMAs consume them) while this slice's
//     MFMAs run; the barrier sits before the last slice's MFMAs, whose phase
//     also reads the next stage's first slice and issues the ring's loads
//     one per MFMA (issued back to back they held the wave's in-order issue);
//   * in LDS, tile row r's 16-byte chunk c sits in slot c ^ ((r >> 1) & 7), so
//     the fragment reads (16 rows per 16 lanes) fall in distinct banks; a
//     direct load writes its lanes in order, so each lane fetches the global
//     chunk that belongs in its slot;
//   * each tile is a buffer resource of its valid rows: rows past the matrix
//     read as zero (their outputs are never stored), and past the last step
//     the ring's loads are out of range (no memory access);
//   * workgroup b runs on XCD b % 8, so each XCD takes a contiguous range of
//     the tile order, which groups 4 row tiles sweeping the column tiles:
//     the tiles one XCD runs together share x and W slices in its L2;
//   * the epilogue goes through LDS so that each lane stores 16 bytes (8 bf16
//     of q_I), with narrow stores only where a piece meets the q_I / w border
//     or the matrix edge.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ix {

namespace {

constexpr int kBK = 64;                  // K per step: 128 bytes of each row
constexpr int kThreads = 256;
constexpr int kGroupM = 4;
constexpr int kXcds = 8;                 // accelerator complex dies; workgroups alternate among them
constexpr int kFewRows = 128;            // up to this many rows: 64 x 64 tiles, 8 stages deep

typedef __attribute__((address_space(3))) void* lds_ptr_t;
// buffer resource word 3 for raw (unformatted, unswizzled) 32-bit data on CDNA
constexpr int kRsrcWord3 = 0x00020000;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int BM, int BN, int STAGES>
__global__ __launch_bounds__(kThreads, 1) void indexer_project_kernel(ProjArgs a) {
  static_assert(BM % 64 == 0 && BN % 64 == 0, "32-row blocks per wave half");
  static_assert(STAGES >= 2, "a stage read while the next lands");
  constexpr int MB = BM / 64, NB = BN / 64;             // 32 x 32 blocks per wave
  constexpr int kStage = (BM + BN) * kBK * 2;           // bytes of one stage
  constexpr int kInst = (BM + BN) / 8 / 4;              // 1 KB loads per wave per stage
  static_assert(kInst % (MB + NB) == 0, "whole loads per fragment read");
  constexpr int kLoadsPerRead = kInst / (MB + NB);
  static_assert((STAGES - 1) * kInst <= 63, "vmcnt counts the ring's loads");
  extern __shared__ __align__(16) unsigned char smem[]; // [STAGES][x rows, W rows][128 B]

  const int tid = threadIdx.x, l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // tile of this workgroup: XCD-contiguous ranges of the grouped tile order
  const int n_m = (int)((a.M + BM - 1) / BM), n_n = (a.N + BN - 1) / BN;
  const int T = n_m * n_n, per = T / kXcds, rem = T % kXcds;
  const int xcd = blockIdx.x % kXcds, li = blockIdx.x / kXcds;
  const int pid = xcd * per + min(xcd, rem) + li, in_group = kGroupM * n_n;
  const int first_m = (pid / in_group) * kGroupM;
  const int gsize = min(n_m - first_m, kGroupM);
  const int tm = first_m + (pid % in_group) % gsize;
  const int tn = (pid % in_group) / gsize;
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;
  const int rows_x = (int)min<int64_t>(BM, a.M - m0), rows_w = min(BN, a.N - n0);

  // loads: this wave's instruction j covers tile rows 8 i .. 8 i + 7 of the
  // stacked [x tile; W tile] (i = wave + 4 j); lane l fills row 8 i + l / 8,
  // slot l % 8, whose chunk is slot ^ (row / 2 % 8) = slot ^ (4 (i % 2) + l / 16)
  const uint32_t row_bytes = (uint32_t)a.K * 2u;
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.x + m0 * a.K), (short)0, (int)((uint32_t)rows_x * row_bytes), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.w + (int64_t)n0 * a.K), (short)0, (int)((uint32_t)rows_w * row_bytes), kRsrcWord3);
  uint32_t off[kInst];
#pragma unroll
  for (int j = 0; j < kInst; ++j) {
    const int i = wave + 4 * j;
    const int r = (i < BM / 8 ? i : i - BM / 8) * 8 + (l >> 3);
    const int c = (l & 7) ^ (4 * (wave & 1) + (l >> 4));
    off[j] = (uint32_t)r * row_bytes + (uint32_t)c * 16u;
  }
  // load j of step kt into its stage; real == false sets bit 31 of every
  // lane's offset, past any tile's range (2^31 bytes at most), so the load
  // touches no memory and only writes zeros
  auto load = [&](int j, int kt, bool real) {
    const int i = wave + 4 * j;
    unsigned char* st = smem + (kt % STAGES) * kStage;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(i < BM / 8 ? xr : wr, (lds_ptr_t)(st + i * 1024), 16,
                                             (int)(off[j] | (real ? 0u : 0x80000000u)), kt * (kBK * 2), 0, 0);
  };

  // compute: wave (wm, wn) owns rows (BM/2) wm .. and columns (BN/2) wn .. of
  // the tile; lane (i32 = l % 32, g = l / 32) supplies row i32's k values
  // 16 ks + 8 g .. + 8 of each fragment, chunk (2 ks + g), at slot
  // (2 ks + g) ^ (i32 / 2 % 8) = 2 ks ^ t with t = g ^ (i32 / 2 % 8)
  const int wm = wave >> 1, wn = wave & 1, i32 = l & 31, kg = l >> 5;
  const int t = kg ^ ((i32 >> 1) & 7);
  const uint32_t a_lane = (uint32_t)(wm * (BM / 2) + i32) * 128u;
  const uint32_t b_lane = (uint32_t)(BM + wn * (BN / 2) + i32) * 128u;
  f32x16 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x16{};
  auto a_frag = [&](const unsigned char* st, int ks, int mb) {
    return *reinterpret_cast<const bf16x8*>(st + ((uint32_t)(t ^ (2 * ks)) << 4) + a_lane + mb * 32 * 128);
  };
  auto b_frag = [&](const unsigned char* st, int ks, int nb) {
    return *reinterpret_cast<const bf16x8*>(st + ((uint32_t)(t ^ (2 * ks)) << 4) + b_lane + nb * 32 * 128);
  };
  // fragment read g of slice ks, in the order the MFMAs consume them:
  // A block 0, then B blocks 0 .. NB - 1, then A blocks 1 .. MB - 1
  auto read_frag = [&](const unsigned char* st, int ks, int g, bf16x8 (&af)[MB], bf16x8 (&bf)[NB]) {
    if (g == 0) af[0] = a_frag(st, ks, 0);
    else if (g <= NB) bf[g - 1] = b_frag(st, ks, g - 1);
    else af[g - NB] = a_frag(st, ks, g - NB);
  };
  auto mfmas = [&](const bf16x8 (&ua)[MB], const bf16x8 (&ub)[NB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ua[mb], ub[nb], acc[mb][nb], 0, 0, 0);
  };
  // one phase: slice ks of stage st is read into (ra, rb) while the MFMAs of
  // (ua, ub) run; LDS reads complete in issue order, so a phase's MFMAs wait
  // only for the previous phase's reads.  With kt_load >= 0 the phase also
  // issues that step's loads, in program order between the reads (the loads
  // write LDS, so the scheduler keeps LDS accesses in program order).
  auto phase = [&](const unsigned char* st, int ks, bf16x8 (&ra)[MB], bf16x8 (&rb)[NB],
                   const bf16x8 (&ua)[MB], const bf16x8 (&ub)[NB], int kt_load = -1, bool real = false) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < MB + NB; ++g) {
      read_frag(st, ks, g, ra, rb);
      if (kt_load >= 0) {
#pragma unroll
        for (int h = 0; h < kLoadsPerRead; ++h) load(kLoadsPerRead * g + h, kt_load, real);
      }
    }
    mfmas(ua, ub);
    if constexpr (MB * NB >= 2 * (MB + NB)) {
      // one read (and its loads) per MB NB / (MB + NB) MFMAs
      constexpr int per = MB * NB / (MB + NB);
#pragma unroll
      for (int g = 0; g < MB + NB; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int m = 0; m < per; ++m) {
          if (kt_load >= 0 && m < kLoadsPerRead) __builtin_amdgcn_sched_group_barrier(0x270, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Every step issues kInst loads per wave (empty ones past the last step),
  // so before a step's barrier the next step has landed once at most the
  // (STAGES - 2) kInst loads of the steps after it are in flight.
  const int KT = a.K / kBK;
  for (int kt = 0; kt < STAGES; ++kt)
#pragma unroll
    for (int j = 0; j < kInst; ++j) load(j, kt, kt < KT);
  wait_vmcnt<(STAGES - 1) * kInst>();
  lds_barrier();
  if constexpr (MB == 1 && NB == 1) {
    // One 32 x 32 block per wave: a step is only 4 MFMAs, so instead of
    // phases the whole next step's fragments are read (with the ring's
    // loads) before this step's MFMAs, behind one barrier: when it passes,
    // every wave's reads of step kt are complete (stage kt is free for step
    // kt + STAGES) and step kt + 1 has landed.
    bf16x8 f[2][4][2];                               // [buffer][slice][A, B]
    f32x16 acc1 = f32x16{};                          // odd slices: two independent MFMA chains
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      f[0][ks][0] = a_frag(smem, ks, 0);
      f[0][ks][1] = b_frag(smem, ks, 0);
    }
    auto step = [&](int kt, bf16x8 (&cur)[4][2], bf16x8 (&nxt)[4][2]) {
      wait_vmcnt<(STAGES - 2) * kInst>();
      lds_barrier();
      const unsigned char* st = smem + ((kt + 1) % STAGES) * kStage;   // stale in the last step, never used
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        nxt[ks][0] = a_frag(st, ks, 0);
        nxt[ks][1] = b_frag(st, ks, 0);
        load(ks, kt + STAGES, kt + STAGES < KT);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ks += 2) {
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur[ks][0], cur[ks][1], acc[0][0], 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur[ks + 1][0], cur[ks + 1][1], acc1, 0, 0, 0);
      }
    };
    static_assert(kInst == 4, "one load per slice");
    int kt = 0;
    for (; kt + 1 < KT; kt += 2) {
      step(kt, f[0], f[1]);
      step(kt + 1, f[1], f[0]);
    }
    if (kt < KT) step(kt, f[0], f[1]);
    acc[0][0] += acc1;
  } else {
    // Step kt reads stage kt % STAGES and enters with its slice 0 in fa.
    // After slice 3's fragments are read every wave is done with that stage,
    // so the barrier goes there; past it, step kt + STAGES loads into the
    // stage, and slice 0 of step kt + 1 is read while slice 3's MFMAs run.
    bf16x8 fa[MB], fb[NB], ga[MB], gb[NB];
#pragma unroll
    for (int g = 0; g < MB + NB; ++g) read_frag(smem, 0, g, fa, fb);
    for (int kt = 0; kt < KT; ++kt) {
      const unsigned char* st = smem + (kt % STAGES) * kStage;
      phase(st, 1, ga, gb, fa, fb);
      phase(st, 2, fa, fb, ga, gb);
      phase(st, 3, ga, gb, fa, fb);
      wait_vmcnt<(STAGES - 2) * kInst>();
      lds_barrier();
      // (in the last step this reads a stale stage, never used)
      phase(smem + ((kt + 1) % STAGES) * kStage, 0, fa, fb, ga, gb, kt + STAGES, kt + STAGES < KT);
    }
  }
  wait_vmcnt<0>();                                  // the empty loads too, before the epilogue's LDS use

  // epilogue, one 32-row block (mb) at a time through a wave-private LDS
  // region of fp32 rows (stride kEpiStride floats: the two 32-lane halves,
  // 4 rows apart, land in disjoint banks): accumulator element e of block
  // (mb, nb) is row 8 (e / 4) + 4 g + e % 4, column nb * 32 + i32; read back,
  // lane l owns 8 consecutive columns of a row and stores them as one 16-byte
  // bf16 piece (or 2-byte / fp32 stores where the piece meets the q_I / w
  // border, the matrix edge or an unaligned q_I)
  constexpr int kWaveCols = BN / 2;
  constexpr int kEpiStride = kWaveCols + 8;
  static_assert(4 * 32 * kEpiStride * 4 <= STAGES * kStage, "epilogue fits the stages");
  static_assert((4 * kEpiStride) % 64 == 32, "halves in disjoint banks");
  static_assert(32 * kWaveCols / 8 % 64 == 0, "whole passes of 8-column pieces");
  float* epi = reinterpret_cast<float*>(smem) + wave * 32 * kEpiStride;
  const int nw = a.N - a.Nq;
  const bool q_vec = ((a.Nq & 7) == 0) && ((reinterpret_cast<uintptr_t>(a.q) & 15) == 0);
  const int c8 = (l % (kWaveCols / 8)) * 8;
  const int col = n0 + wn * kWaveCols + c8;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        epi[(8 * (e >> 2) + 4 * kg + (e & 3)) * kEpiStride + nb * 32 + i32] = acc[mb][nb][e];
    wave_lds_sync();
#pragma unroll
    for (int it = 0; it < 32 * kWaveCols / 8 / 64; ++it) {
      const int r = (l + 64 * it) / (kWaveCols / 8);
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(epi + r * kEpiStride + c8);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(epi + r * kEpiStride + c8 + 4);
      const int64_t row = m0 + wm * (BM / 2) + mb * 32 + r;
      if (row >= a.M) continue;
      if (q_vec && col + 8 <= a.Nq) {
        u32x4 p;
        p[0] = pack_bf16x2(v0[0], v0[1]);
        p[1] = pack_bf16x2(v0[2], v0[3]);
        p[2] = pack_bf16x2(v1[0], v1[1]);
        p[3] = pack_bf16x2(v1[2], v1[3]);
        *reinterpret_cast<u32x4*>(a.q + row * a.Nq + col) = p;
      } else {
        const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int cj = col + j;
          if (cj < a.Nq) a.q[row * a.Nq + cj] = (uint16_t)bf16_rne(v[j]);
          else if (cj < a.N) a.wo[row * nw + (cj - a.Nq)] = v[j];
        }
      }
    }
    wave_lds_sync();
  }
}

template <int BM, int BN, int STAGES>
hipError_t launch_tiles(const ProjArgs& a, hipStream_t s) {
  // a tile's buffer resource spans at most 2^31 bytes
  if ((int64_t)a.K * 2 * (BM > BN ? BM : BN) > (int64_t)INT32_MAX) return hipErrorInvalidValue;
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  if (tiles > (int64_t)INT32_MAX) return hipErrorInvalidValue;
  const size_t lds = (size_t)STAGES * (BM + BN) * kBK * 2;
  auto* k = &indexer_project_kernel<BM, BN, STAGES>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3((unsigned)tiles), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_project(const ProjArgs& a, hipStream_t s) {
  if (a.M < 0 || a.N <= 0 || a.K <= 0 || a.K % kBK != 0 || a.Nq < 0 || a.Nq > a.N) return hipErrorInvalidValue;
  if (a.M == 0) return hipSuccess;
  if (a.M <= kFewRows) return launch_tiles<64, 64, 8>(a, s);
  return launch_tiles<256, 256, 2>(a, s);
}

}  // namespace ix

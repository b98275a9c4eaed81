// gemm.hip -- INT8 x INT8 -> INT32 GEMM with a fused FP32 dequantization
// epilogue, for gfx950 (CDNA4) matrix cores.
//
// What is computed ("feat(mps): support MiniMax-H3 INT8 inference on Apple
// M5", LightX2V pull request #1672, description and commit notes): the
// projection of per-token INT8 activations A[M,K] by INT8 weights W[N,K],
// consumed in the Linear's stored layout without repacking and without
// dequantizing W, with K an exact multiple of the K tile (no K padding).
// The epilogue computes ((float)acc * sa[m]) * sw[n] + bias[n] in binary32,
// bias added before the single BF16 rounding ("MLX implementation and
// experiment report", "What the default preserves").
//
// Design (gfx950):
//   * Block tile BM tokens x BN channels, K staged BK bytes at a time through
//     LDS, double buffered.  Tiles are filled with buffer_load_dwordx4 ... lds
//     (direct global -> LDS, 16 bytes per lane), so staging costs no VGPRs.
//     The buffer form, through one buffer resource per operand tile, rather
//     than the global form: the compiler treats an outstanding global (flat)
//     load into LDS as touching both memory and LDS and then waits for every
//     LDS read (lgkmcnt(0)) before each use of a fragment; with buffer loads
//     its fragment waits count only the reads a k-step still needs.
//   * LDS rows are BK bytes; the 16-byte chunk c of row r sits at position
//     c ^ swz(r), which makes the wave's 16-byte fragment reads free of bank
//     conflicts whether the LDS serves 8 lanes x 16 B (32 banks) or
//     16 lanes x 16 B (64 banks) per cycle.  The direct loads write whole
//     1 KiB runs, so the swizzle is applied on the global-address side.
//   * v_mfma_i32_32x32x32_i8: weights are the MFMA "A" operand and tokens the
//     "B" operand, so each lane's accumulators hold 4 consecutive output
//     channels of one token -> 8-byte BF16 stores.
//   * Tokens beyond M and channels beyond N are loaded from a clamped row (no
//     out-of-range reads) and never stored.
//   * Tile order: the hardware deals workgroups round-robin to the 8 XCDs;
//     block ids are remapped so each XCD owns a contiguous run of tiles, and
//     that run is walked in groups of GROUP_M token tiles so the tiles in
//     flight on one XCD share A rows and W rows in its L2.
//   * Split-K (skinny M): grid.z slices the K stages; each slice writes INT32
//     partials to the workspace and a second kernel sums them (integer sums
//     are exact in any order) and applies the epilogue.
#include "internal.h"

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <unordered_map>

#pragma clang fp contract(off)

namespace w8a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kXcds = 8;
constexpr int EPI_PARTIAL = 3;       // split-K slice: raw INT32, [M,N] layout
constexpr int EPI_PARTIAL_TILE = 4;  // tail split-K slice: raw INT32 per tile

template <int BM_, int BN_, int BK_, int WGM_, int WGN_, int GROUP_M_,
          int NS_>
struct Cfg {
  static constexpr int BM = BM_;   // tokens per block tile
  static constexpr int BN = BN_;   // output channels per block tile
  static constexpr int BK = BK_;   // K bytes per LDS stage
  static constexpr int WGM = WGM_; // waves along M
  static constexpr int WGN = WGN_; // waves along N
  static constexpr int GROUP_M = GROUP_M_;
  static constexpr int NS = NS_;   // LDS stages in the ring
  static constexpr int WAVES = WGM * WGN;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int WM = BM / WGM;  // tokens per wave
  static constexpr int WN = BN / WGN;  // channels per wave
  static constexpr int TM = WM / 32;   // 32x32 MFMA tiles per wave, tokens
  static constexpr int TN = WN / 32;   // ... channels
  static constexpr int CPR = BK / 16;  // 16-byte chunks per LDS row
  static constexpr int A_BYTES = BM * BK;
  static constexpr int B_BYTES = BN * BK;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS = NS * STAGE;
  static constexpr int KS = BK / 32;  // MFMA k-steps per stage
  // BF16 epilogue staged through LDS (needs 128-channel waves and room for
  // the whole BM x BN BF16 tile in the ring).
  static constexpr bool STAGED_EPI = (WN == 128) && (BM * BN * 2 <= LDS);
  static constexpr int A_LOADS = A_BYTES / (1024 * WAVES);  // per wave
  static constexpr int B_LOADS = B_BYTES / (1024 * WAVES);
  static_assert(BK == 64 || BK == 128, "BK");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile");
  static_assert(A_BYTES % (1024 * WAVES) == 0, "A staging");
  static_assert(B_BYTES % (1024 * WAVES) == 0, "B staging");
  static_assert(LDS <= 160 * 1024, "LDS");
  // Two slots: each stage's slot is refilled with the stage after next at
  // its last k-step.  Three or more: the previous stage's slot is refilled,
  // and up to NS-2 stages stay in flight behind the one waited for.
  static_assert(NS >= 2 && NS <= 6, "stages");
  static_assert((A_BYTES + B_BYTES) / (1024 * WAVES) * (NS >= 3 ? NS - 2 : 1) <=
                    63,
                "vmcnt counts at most 63 outstanding loads");
  static_assert(KS % 2 == 0, "fragment double buffering alternates per k-step");
};

// Position of logical 16-byte chunk c in LDS row r (an involution in c).
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  if (CPR == 4) return c ^ (((r >> 1) ^ (r >> 3)) & 3);
  return c ^ (((r >> 1) ^ ((r & 1) << 2)) & 7);
}

// 16 bytes per lane from buffer `r` at byte voff + soff into LDS at `l`
// (lane i's bytes at l + 16 i).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, int voff,
                                           int soff, lds_void *l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, voff, soff, 0, 0);
}

// A raw buffer resource (no stride, no swizzle) over [base, base + 2^31 - 1)
// bytes.  The address is first made wave-uniform: readfirstlane returns a
// signed int, so each 32-bit half is widened through uint32_t (a sign
// extension of the low half would corrupt the high half).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const int8_t *base) {
  const uint64_t ad = (uint64_t)(uintptr_t)base;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ad);
  const uint64_t hi =
      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(ad >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)((hi << 32) | lo),
                                           (short)0, 0x7fffffff, 0x00020000);
}

// Four consecutive channel scales (biases) from channel n, a multiple of 4:
// one vector load when the array is 16-byte (8-byte) aligned, else one
// load per value (the boundary accepts 4-byte aligned scales and 2-byte
// aligned biases, e.g. a channel slice of larger arrays).  `vec` is uniform
// across the launch.
__device__ __forceinline__ float4 load_scale4(const float *sw, int n,
                                              bool vec) {
  if (vec) return *reinterpret_cast<const float4 *>(sw + n);
  return make_float4(sw[n], sw[n + 1], sw[n + 2], sw[n + 3]);
}

__device__ __forceinline__ float4 load_bias4(const uint16_t *b, int n,
                                             bool vec) {
  uint32_t b01, b23;
  if (vec) {
    const uint2 v = *reinterpret_cast<const uint2 *>(b + n);
    b01 = v.x;
    b23 = v.y;
  } else {
    b01 = (uint32_t)b[n] | ((uint32_t)b[n + 1] << 16);
    b23 = (uint32_t)b[n + 2] | ((uint32_t)b[n + 3] << 16);
  }
  return make_float4(bf16_to_f32(b01 & 0xFFFFu), bf16_to_f32(b01 >> 16),
                     bf16_to_f32(b23 & 0xFFFFu), bf16_to_f32(b23 >> 16));
}

__device__ __forceinline__ v4i read_lds16(const int8_t *lds_base, int off) {
  return *reinterpret_cast<const v4i *>(lds_base + off);
}

// The hardware deals workgroups round-robin to the 8 XCDs; remap block id
// `bid` of a T-block grid so that each XCD owns a contiguous run of tile
// indices.
__device__ __forceinline__ int xcd_remap(int bid, int T) {
  const int xcd = bid % kXcds;
  const int local = bid / kXcds;
  const int per = T / kXcds, rem = T % kXcds;
  return xcd * per + min(xcd, rem) + local;
}

// Tile index -> (token tile, channel tile): groups of `group_m` token tiles
// sweep all channel tiles, token tile fastest within a group, so tiles in
// flight together share A rows and W rows.
__device__ __forceinline__ void grouped_tile(int L, int tiles_m, int tiles_n,
                                             int group_m, int &tm, int &tn) {
  const int span = group_m * tiles_n;
  const int g = L / span;
  const int first = g * group_m;
  const int gsize = min(tiles_m - first, group_m);
  const int within = L - g * span;
  tm = first + within % gsize;
  tn = within / gsize;
}

// Wait until this wave's direct loads of one stage have landed in LDS.
// Loads complete in issue order, so it suffices that no more than the loads
// of the `later` stages requested after it remain outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// s_waitcnt immediate for gfx9-family: vmcnt in bits [3:0] and [15:14],
// expcnt [6:4], lgkmcnt [11:8]; unconstrained counters at their maximum.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 0xF) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}

// Wait until at most N LDS reads of this wave are outstanding.  The builtin
// (rather than inline asm) lets the compiler's own wait insertion see it;
// the scheduling barriers keep the surrounding reads and MFMAs in order.
template <int N>
__device__ __forceinline__ void wait_lgkm() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, N));
}

// Workgroup barrier without the memory fences of __syncthreads (which would
// also wait for every outstanding direct load); ordering of LDS data is
// handled by the explicit vmcnt waits above.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct KernelArgs {
  const int8_t *a;
  const float *sa;
  const int8_t *w;
  const float *sw;
  const uint16_t *bias;
  void *out;
  int M, N, K;
  int tiles_m, tiles_n;
  int stages_total;  // K / BK
  int splits;
  int group_m;
  int tile_base;     // first tile index of this launch
  int remap;         // 1: XCD remap of block ids over the grid
  int vec_sw;        // 1: sw is 16-byte aligned (vector loads)
  int vec_bias;      // 1: bias is 8-byte aligned (vector loads)
};

template <class C, int EPI>
__global__ __launch_bounds__(C::THREADS, 1) void gemm_kernel(KernelArgs p) {
  extern __shared__ __attribute__((aligned(1024))) int8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave / C::WGN;
  const int wave_n = wave % C::WGN;

  int tm, tn;
  const int L = p.remap ? xcd_remap(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  grouped_tile(p.tile_base + L, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * C::BM;
  const int n0 = tn * C::BN;

  // K stages of this split.
  const int z = blockIdx.z;
  const int kt0 = (int)((int64_t)z * p.stages_total / p.splits);
  const int kt1 = (int)((int64_t)(z + 1) * p.stages_total / p.splits);
  const int nk = kt1 - kt0;

  // Direct loads: a uniform base per operand, advanced by BK bytes per
  // stage, plus a 32-bit per-lane offset per load instruction (the row in
  // the tile, clamped to the last valid row, times K, plus the chunk that
  // lands in this lane's 16 LDS bytes).  Row offsets plus the stage offset
  // stay below 257 * W8A8_MAX_K, far inside the 2^31 - 1 bytes of the
  // buffer resource below.
  const int8_t *a_base = p.a + (int64_t)m0 * p.K + (int64_t)kt0 * C::BK;
  const int8_t *b_base = p.w + (int64_t)n0 * p.K + (int64_t)kt0 * C::BK;
  int oa[C::A_LOADS], ob[C::B_LOADS];
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) {
    const int slot = (j * C::WAVES + wave) * 64 + lane;
    const int r = slot / C::CPR;
    const int c = swz<C::CPR>(r, slot % C::CPR);
    oa[j] = min(r, p.M - 1 - m0) * p.K + c * 16;
  }
#pragma unroll
  for (int j = 0; j < C::B_LOADS; ++j) {
    const int slot = (j * C::WAVES + wave) * 64 + lane;
    const int r = slot / C::CPR;
    const int c = swz<C::CPR>(r, slot % C::CPR);
    ob[j] = min(r, p.N - 1 - n0) * p.K + c * 16;
  }

  // One buffer resource per operand over this tile's rows; a load's byte
  // offset is its lane offset above plus the stage's BK * src.
  const auto ra = tile_rsrc(a_base);
  const auto rb = tile_rsrc(b_base);

  // Request stage `src` of this split into ring slot `slot`.
  auto issue_into = [&](int slot, int src) {
    const int soff = __builtin_amdgcn_readfirstlane(src * C::BK);
    int8_t *sa_base = smem + slot * C::STAGE;
    int8_t *sb_base = sa_base + C::A_BYTES;
#pragma unroll
    for (int j = 0; j < C::A_LOADS; ++j)
      load_lds16(ra, oa[j], soff,
                 (lds_void *)(sa_base + (j * C::WAVES + wave) * 1024));
#pragma unroll
    for (int j = 0; j < C::B_LOADS; ++j)
      load_lds16(rb, ob[j], soff,
                 (lds_void *)(sb_base + (j * C::WAVES + wave) * 1024));
  };

  // Fragment reads: lane reads 16 bytes of row (lane & 31) of each 32-row
  // fragment, logical chunk 2*ks + (lane >> 5) of the stage, at its swizzled
  // position.  Fragment rows start at multiples of 32, where the swizzle
  // repeats, so one per-lane offset per k-step serves every fragment.
  const int frow = lane & 31;
  const int fchunk = lane >> 5;
  int rx[C::KS], rw[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const int r1 = wave_m * C::WM + frow;
    const int r2 = wave_n * C::WN + frow;
    rx[ks] = r1 * C::BK + swz<C::CPR>(r1, ks * 2 + fchunk) * 16;
    rw[ks] = C::A_BYTES + r2 * C::BK + swz<C::CPR>(r2, ks * 2 + fchunk) * 16;
  }
  v4i fx[2][C::TM], fw[2][C::TN];
  auto read_frags = [&](int buf, int ks, v4i *xa, v4i *wb) {
    const int8_t *base = smem + buf * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
      xa[i] = read_lds16(base, rx[ks] + i * 32 * C::BK);
#pragma unroll
    for (int i = 0; i < C::TN; ++i)
      wb[i] = read_lds16(base, rw[ks] + i * 32 * C::BK);
  };

  v16i acc[C::TN][C::TM];
#pragma unroll
  for (int i = 0; i < C::TN; ++i)
#pragma unroll
    for (int j = 0; j < C::TM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  // Ring of NS stages.  Fragment registers are double buffered across
  // k-steps: the reads of k-step s+1 are interleaved with the MFMAs of
  // k-step s, and the last k-step of stage kt reads k-step 0 of stage kt+1.
  // At the start of that last k-step the wave waits until stage kt+1 has
  // landed and all waves meet at a barrier; then one stage is requested:
  //  * NS = 2 (the large configuration, 128-byte stages): every read of
  //    stage kt has been issued by then; once they have completed (waited
  //    for before the barrier) its slot takes stage kt+2, which then has
  //    one stage time to land.
  //  * NS >= 3: stages 0..NS-2 are requested up front and the barrier means
  //    every read of stage kt-1's slot is done; that slot takes stage
  //    kt+NS-1, and NS-3 stages stay in flight behind stage kt+1.
  // In both cases the number of loads in flight at the wait is a constant,
  // so the steady-state loop body is straight-line code.
  constexpr int LOADS = C::A_LOADS + C::B_LOADS;  // per wave per stage
  constexpr int READS = C::TM + C::TN;            // per k-step per wave
  constexpr int MFMAS = C::TM * C::TN;            // per k-step per wave
  auto mfma_step = [&](const v4i *xa, const v4i *wb) {
#pragma unroll
    for (int i = 0; i < C::TN; ++i)
#pragma unroll
      for (int j = 0; j < C::TM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wb[i], xa[j],
                                                          acc[i][j], 0, 0, 0);
  };
  // Interleave: after every MFMAS/READS MFMAs, one fragment read.
  auto interleave = [&]() {
#pragma unroll
    for (int r = 0; r < READS; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, MFMAS / READS, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (MFMAS % READS != 0)
      __builtin_amdgcn_sched_group_barrier(0x008, MFMAS % READS, 0);
  };
  // One stage: its KS k-steps; the last one crosses into stage kt+1.
  // Every stage but the last requests one stage's loads after its barrier:
  // the stage due while it exists, otherwise a second copy of the last
  // stage into the free slot (harmless, and it keeps the number of loads in
  // flight constant, so the loop has one body and one wait count).
  auto stage = [&](int kt, bool last) {
    const int buf = kt % C::NS;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int cur = ks & 1;
      // Code does not move across k-steps: that would keep three fragment
      // sets live and spill.
      __builtin_amdgcn_sched_barrier(0);
      if (ks + 1 < C::KS) {
        read_frags(buf, ks + 1, fx[cur ^ 1], fw[cur ^ 1]);
        mfma_step(fx[cur], fw[cur]);
        interleave();
      } else if (!last) {
        if constexpr (C::NS == 2) {
          wait_lgkm<0>();   // this wave's reads of stage kt are done
          wait_vmcnt<0>();  // stage kt+1 has landed
          block_barrier();
          issue_into(kt % 2, min(kt + 2, nk - 1));
        } else {
          wait_vmcnt<(C::NS - 3) * LOADS>();
          block_barrier();
          issue_into((kt + C::NS - 1) % C::NS, min(kt + C::NS - 1, nk - 1));
        }
        read_frags((kt + 1) % C::NS, 0, fx[cur ^ 1], fw[cur ^ 1]);
        mfma_step(fx[cur], fw[cur]);
        interleave();
      } else {
        mfma_step(fx[cur], fw[cur]);
      }
    }
  };
  // Prologue: stages 0 and 1 (NS = 2) or 0..NS-2 (a missing stage is
  // replaced by a copy of the last one, as above), then wait for stage 0.
  // (The host plans at least 512 bytes of K per split; a split without
  // stages skips the pipeline and stores zero accumulators.)
  if (nk > 0) {
    if constexpr (C::NS == 2) {
      issue_into(0, 0);
      issue_into(1, min(1, nk - 1));
      wait_vmcnt<LOADS>();
    } else {
#pragma unroll
      for (int s = 0; s < C::NS - 1; ++s) issue_into(s, min(s, nk - 1));
      wait_vmcnt<(C::NS - 2) * LOADS>();
    }
    block_barrier();
    read_frags(0, 0, fx[0], fw[0]);
    for (int kt = 0; kt + 1 < nk; ++kt) stage(kt, false);
    stage(nk - 1, true);
  }
  // The drain copies may still be landing in LDS: they must have landed
  // before the epilogue reuses the ring or the work group releases it.
  wait_vmcnt<0>();

  // Epilogue.  Lane holds token m = base + (lane & 31) and, for register
  // 4g + t, channel n = base + 8g + 4*(lane >> 5) + t.
  if constexpr (EPI == EPI_BF16 && C::STAGED_EPI) {
    // BF16 results go through LDS so that the global stores write whole
    // row segments (16 lanes x 16 B = 256 contiguous bytes per row) rather
    // than 32 rows x 16 B per instruction.  Each wave stages its WM x WN
    // block row-major in its own LDS region; 16-byte chunk c of row r sits
    // at chunk c ^ (r mod CPRW) and its 8-byte halves are swapped when bit 4
    // of r is set, which keeps both the 8-byte writes (32 rows per half
    // wave) and the 16-byte reads free of bank conflicts.
    constexpr int ROWB = C::WN * 2;    // bytes per staged row
    constexpr int CPRW = ROWB / 16;    // 16-byte chunks per staged row
    constexpr int RPI = 64 / CPRW;     // staged rows per wave read
    block_barrier();  // every wave is done reading the ring
    int8_t *region = smem + wave * (C::WM * ROWB);
    const int mb = m0 + wave_m * C::WM;
    const int nb = n0 + wave_n * C::WN;
    // N is a multiple of 128 and so is nb: a wave's 128 channels are all
    // inside N or all past it (then nothing of this wave is stored).
    // Two copies of the arithmetic, with and without the bias add, so that
    // neither carries a per-channel test.
    auto stage_rows = [&](auto with_bias) {
      constexpr bool kBias = decltype(with_bias)::value;
      float sam[C::TM];
#pragma unroll
      for (int j = 0; j < C::TM; ++j) {
        const int m = mb + j * 32 + (lane & 31);
        sam[j] = m < p.M ? p.sa[m] : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < C::TN; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int nl = i * 32 + 8 * g + 4 * (lane >> 5);
          const int n = nb + nl;
          const float4 swn = load_scale4(p.sw, n, p.vec_sw);
          float4 bv;
          if constexpr (kBias) bv = load_bias4(p.bias, n, p.vec_bias);
          const int c = nl >> 3, h = (nl >> 2) & 1;
#pragma unroll
          for (int j = 0; j < C::TM; ++j) {
            float t0 = ((float)acc[i][j][4 * g + 0] * sam[j]) * swn.x;
            float t1 = ((float)acc[i][j][4 * g + 1] * sam[j]) * swn.y;
            float t2 = ((float)acc[i][j][4 * g + 2] * sam[j]) * swn.z;
            float t3 = ((float)acc[i][j][4 * g + 3] * sam[j]) * swn.w;
            if constexpr (kBias) {
              t0 = t0 + bv.x;
              t1 = t1 + bv.y;
              t2 = t2 + bv.z;
              t3 = t3 + bv.w;
            }
            const int r = j * 32 + (lane & 31);
            const int off = r * ROWB + ((c ^ (r & (CPRW - 1))) << 4) +
                            ((h ^ ((r >> 4) & 1)) << 3);
            *reinterpret_cast<uint2 *>(region + off) =
                make_uint2(pack_bf16x2(t0, t1), pack_bf16x2(t2, t3));
          }
        }
      }
    };
    if (nb < p.N) {
      if (p.bias)
        stage_rows(std::true_type{});
      else
        stage_rows(std::false_type{});
    }
    uint16_t *out = static_cast<uint16_t *>(p.out);
#pragma unroll 4
    for (int it = 0; it < C::WM / RPI; ++it) {
      const int r = it * RPI + lane / CPRW;
      const int c = lane % CPRW;
      v4i v = *reinterpret_cast<const v4i *>(region + r * ROWB +
                                             ((c ^ (r & (CPRW - 1))) << 4));
      if ((r >> 4) & 1) v = v4i{v.z, v.w, v.x, v.y};
      const int m = mb + r, n = nb + c * 8;
      if (m < p.M && n < p.N)
        *reinterpret_cast<v4i *>(out + (int64_t)m * p.N + n) = v;
    }
    return;
  }
  if constexpr (EPI == EPI_PARTIAL_TILE) {
    // Raw accumulators of this K slice in a tile-local block of the
    // workspace (slice z of tail tile blockIdx.x), in register order: the
    // 4-register group g of accumulator (i, j) of wave w is one 1 KiB run,
    // lane-major, so every store writes whole contiguous lines.  Rows and
    // columns past M or N hold values of clamped rows; the reduction skips
    // them.
    int *dst = static_cast<int *>(p.out) +
               ((int64_t)z * gridDim.x + blockIdx.x) * (C::BM * C::BN) +
               wave * (C::TN * C::TM * 4 * 256) + lane * 4;
#pragma unroll
    for (int i = 0; i < C::TN; ++i)
#pragma unroll
      for (int j = 0; j < C::TM; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<v4i *>(dst + ((i * C::TM + j) * 4 + g) * 256) =
              v4i{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                  acc[i][j][4 * g + 3]};
    return;
  }
  const int64_t MN = (int64_t)p.M * p.N;
#pragma unroll
  for (int j = 0; j < C::TM; ++j) {
    const int m = m0 + wave_m * C::WM + j * 32 + (lane & 31);
    if (m >= p.M) continue;
    float sam = 0.0f;
    if (EPI == EPI_BF16 || EPI == EPI_FP32) sam = p.sa[m];
#pragma unroll
    for (int i = 0; i < C::TN; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wave_n * C::WN + i * 32 + 8 * g + 4 * (lane >> 5);
        if (n >= p.N) continue;
        const int64_t o = (int64_t)m * p.N + n;
        const int acc0 = acc[i][j][4 * g + 0], acc1 = acc[i][j][4 * g + 1];
        const int acc2 = acc[i][j][4 * g + 2], acc3 = acc[i][j][4 * g + 3];
        if (EPI == EPI_I32 || EPI == EPI_PARTIAL) {
          int *dst = static_cast<int *>(p.out) + (EPI == EPI_PARTIAL ? z * MN : 0);
          *reinterpret_cast<v4i *>(dst + o) = v4i{acc0, acc1, acc2, acc3};
          continue;
        }
        const float4 swn = load_scale4(p.sw, n, p.vec_sw);
        float t0 = ((float)acc0 * sam) * swn.x;
        float t1 = ((float)acc1 * sam) * swn.y;
        float t2 = ((float)acc2 * sam) * swn.z;
        float t3 = ((float)acc3 * sam) * swn.w;
        if (p.bias) {
          const float4 bv = load_bias4(p.bias, n, p.vec_bias);
          t0 = t0 + bv.x;
          t1 = t1 + bv.y;
          t2 = t2 + bv.z;
          t3 = t3 + bv.w;
        }
        if (EPI == EPI_FP32) {
          *reinterpret_cast<float4 *>(static_cast<float *>(p.out) + o) =
              make_float4(t0, t1, t2, t3);
        } else {
          uint2 v;
          v.x = pack_bf16x2(t0, t1);
          v.y = pack_bf16x2(t2, t3);
          *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.out) + o) = v;
        }
      }
    }
  }
}

// Sum of split-K INT32 partials + epilogue, 4 outputs per thread.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(
    const int *__restrict__ part, int splits, const float *__restrict__ sa,
    const float *__restrict__ sw, const uint16_t *__restrict__ bias,
    void *__restrict__ out, int M, int N, bool vec_sw, bool vec_bias) {
  const int64_t MN = (int64_t)M * N;
  const int64_t quads = MN / 4;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < quads;
       q += (int64_t)gridDim.x * 256) {
    const int64_t o = q * 4;
    // Up to eight slices' loads in flight at a time (a serial chain of
    // loads would wait out one memory latency per slice).
    v4i s = v4i{0, 0, 0, 0};
    for (int z0 = 0; z0 < splits; z0 += 8) {
      v4i v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v[i] = z0 + i < splits
                   ? *reinterpret_cast<const v4i *>(part + (z0 + i) * MN + o)
                   : v4i{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 8; ++i) s += v[i];
    }
    if (EPI == EPI_I32) {
      *reinterpret_cast<v4i *>(static_cast<int *>(out) + o) = s;
      continue;
    }
    const int m = (int)(o / N);
    const int n = (int)(o - (int64_t)m * N);
    const float sam = sa[m];
    const float4 swn = load_scale4(sw, n, vec_sw);
    float t0 = ((float)s.x * sam) * swn.x;
    float t1 = ((float)s.y * sam) * swn.y;
    float t2 = ((float)s.z * sam) * swn.z;
    float t3 = ((float)s.w * sam) * swn.w;
    if (bias) {
      const float4 bv = load_bias4(bias, n, vec_bias);
      t0 = t0 + bv.x;
      t1 = t1 + bv.y;
      t2 = t2 + bv.z;
      t3 = t3 + bv.w;
    }
    if (EPI == EPI_FP32) {
      *reinterpret_cast<float4 *>(static_cast<float *>(out) + o) =
          make_float4(t0, t1, t2, t3);
    } else {
      uint2 v;
      v.x = pack_bf16x2(t0, t1);
      v.y = pack_bf16x2(t2, t3);
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + o) = v;
    }
  }
}

// Sum of the K slices of the tail tiles + epilogue.  Block b covers tail
// tile b / QB (QB blocks of 256 threads per tile); thread q of the tile
// reads the q-th 16-byte run of each slice (the partial-tile layout above)
// and maps it back to its token row and 4 channels.
template <class C, int EPI>
__global__ __launch_bounds__(256) void tail_reduce_kernel(
    const int *__restrict__ part, int splits, int ntail, int tile_base,
    int tiles_m, int tiles_n, int group_m, const float *__restrict__ sa,
    const float *__restrict__ sw, const uint16_t *__restrict__ bias,
    void *__restrict__ out, int M, int N, bool vec_sw, bool vec_bias) {
  constexpr int QB = C::BM * C::BN / 4 / 256;
  const int t = blockIdx.x / QB;
  const int q = (blockIdx.x % QB) * 256 + threadIdx.x;
  const int lane = q % 64, g = (q / 64) % 4, j = (q / 256) % C::TM;
  const int i = (q / (256 * C::TM)) % C::TN;
  const int wave = q / (256 * C::TM * C::TN);
  const int lm = (wave / C::WGN) * C::WM + j * 32 + (lane & 31);
  const int ln = (wave % C::WGN) * C::WN + i * 32 + 8 * g + 4 * (lane >> 5);
  int tm, tn;
  grouped_tile(tile_base + t, tiles_m, tiles_n, group_m, tm, tn);
  const int m = tm * C::BM + lm, n = tn * C::BN + ln;
  if (m >= M || n >= N) return;
  const int64_t tile_elems = (int64_t)C::BM * C::BN;
  const int *src = part + (int64_t)t * tile_elems + q * 4;
  const int64_t zs = (int64_t)ntail * tile_elems;  // between slices
  v4i s = v4i{0, 0, 0, 0};
  for (int z0 = 0; z0 < splits; z0 += 8) {  // eight slices' loads in flight
    v4i v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      v[i] = z0 + i < splits
                 ? *reinterpret_cast<const v4i *>(src + (z0 + i) * zs)
                 : v4i{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) s += v[i];
  }
  const int64_t o = (int64_t)m * N + n;
  if (EPI == EPI_I32) {
    *reinterpret_cast<v4i *>(static_cast<int *>(out) + o) = s;
    return;
  }
  const float sam = sa[m];
  const float4 swn = load_scale4(sw, n, vec_sw);
  float t0 = ((float)s.x * sam) * swn.x;
  float t1 = ((float)s.y * sam) * swn.y;
  float t2 = ((float)s.z * sam) * swn.z;
  float t3 = ((float)s.w * sam) * swn.w;
  if (bias) {
    const float4 bv = load_bias4(bias, n, vec_bias);
    t0 = t0 + bv.x;
    t1 = t1 + bv.y;
    t2 = t2 + bv.z;
    t3 = t3 + bv.w;
  }
  if (EPI == EPI_FP32) {
    *reinterpret_cast<float4 *>(static_cast<float *>(out) + o) =
        make_float4(t0, t1, t2, t3);
  } else {
    uint2 v;
    v.x = pack_bf16x2(t0, t1);
    v.y = pack_bf16x2(t2, t3);
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + o) = v;
  }
}

// ---------------------------------------------------------------------------
// Single-launch GEMM for at most 64 tokens
// ---------------------------------------------------------------------------
// With so few tokens the weights dominate the bytes (M = 64, K = N = 5376:
// 28.9 MB of 30 MB) and the call is bound by streaming them from HBM.  Each
// work group owns all tokens and 32 output channels over the whole K, so
// no partial sums leave the work group and one launch does the call:
//   * K is staged 256 bytes at a time (8 k-steps of 32 bytes) through a ring
//     of NS LDS slots filled by direct loads (each 1 KiB load instruction
//     covers 4 whole rows of the stage);
//   * wave w of the 8 computes k-step w of every stage: it reads its token
//     and weight fragments from the slot and issues TM MFMAs, so the waves
//     split K and nothing is shared between them but the staging;
//   * the waves' INT32 sums meet in LDS once the ring is drained, and all
//     threads finish the call: 4 outputs each, summed over the 8 waves,
//     then the same epilogue as the tiled kernels.
// Token rows past M are loaded from row M - 1 and never stored.  When K is
// an odd number of 128-byte halves the last stage is half full: its missing
// columns are loaded from the row's last 16 bytes (in bounds) and the waves
// whose k-step lies there skip it.
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyThreads = kSkinnyWaves * 64;
#ifndef W8A8_SKINNY_NS
#define W8A8_SKINNY_NS 4
#endif

template <int TM>
struct SkinnyCfg {
  static constexpr int BK = 256;                 // K bytes per stage
  static constexpr int CPR = BK / 16;            // 16-byte chunks per row
  static constexpr int A_ROWS = 32 * TM;         // token rows staged
  static constexpr int B_ROWS = 32;              // channel rows staged
  static constexpr int STAGE = (A_ROWS + B_ROWS) * BK;
  static constexpr int NS = W8A8_SKINNY_NS;
  static constexpr int LOADS = STAGE / (1024 * kSkinnyWaves);  // per wave
  static constexpr int LDS = NS * STAGE;
  // cross-wave sums: per wave 32*TM tokens x 32 channels of INT32, rows
  // padded by 4 ints so 16-byte stores of 32 rows spread over the banks
  static constexpr int ROW = 32 + 4;
  static constexpr int WAVE = 32 * TM * ROW;
  static_assert(STAGE % (1024 * kSkinnyWaves) == 0, "whole loads per wave");
  static_assert(kSkinnyWaves * WAVE * 4 <= LDS, "sums fit in the ring");
  static_assert(LDS <= 160 * 1024, "LDS");
};

// Position of logical 16-byte chunk c in staged row r (16 chunks per row):
// the 16 lanes that one LDS cycle serves read 16 different rows at one
// logical chunk, which land on 16 different physical chunks.
__device__ __forceinline__ int swz16(int r, int c) { return c ^ (r & 15); }

template <int TM, int EPI>
__global__ __launch_bounds__(kSkinnyThreads, 1) void skinny_kernel(
    KernelArgs p) {
  using C = SkinnyCfg<TM>;
  extern __shared__ __attribute__((aligned(1024))) int8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 32;
  const int halves = p.K / 128;
  const int nst = (halves + 1) / 2;  // stages (the last may be half)

  // Direct loads: instruction j of this wave fills 1 KiB block
  // b = j * 8 + wave of a stage: token rows 4b .. 4b + 3, or, past the
  // token rows, channel rows.  Lane i writes row 4b + i / 16 at physical
  // chunk i mod 16, which holds logical chunk swz16(row, i mod 16).
  int rowoff[C::LOADS], chunk[C::LOADS];
  bool is_w[C::LOADS];
#pragma unroll
  for (int j = 0; j < C::LOADS; ++j) {
    const int b = j * kSkinnyWaves + wave;
    const int r = b * 4 + lane / 16;  // staged row
    is_w[j] = r >= C::A_ROWS;
    // rows relative to the operand's resource base: tokens from row 0,
    // weights from this work group's first channel (offsets stay below
    // 64 * W8A8_MAX_K)
    const int grow = is_w[j] ? r - C::A_ROWS : min(r, p.M - 1);
    rowoff[j] = grow * p.K;
    chunk[j] = swz16(r, lane & 15) * 16;
  }
  const auto ra = tile_rsrc(p.a);
  const auto rw = tile_rsrc(p.w + (int64_t)n0 * p.K);
  auto issue = [&](int slot, int st) {
    int8_t *base = smem + slot * C::STAGE;
    const int s0 = min(st, nst - 1) * C::BK;
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) {
      const int col = min(s0 + chunk[j], p.K - 16);
      load_lds16(is_w[j] ? rw : ra, rowoff[j] + col, 0,
                 (lds_void *)(base + (j * kSkinnyWaves + wave) * 1024));
    }
  };

  // Fragment reads of this wave's k-step: lane reads row (lane mod 32) of a
  // 32-row fragment, logical chunk 2 wave + lane / 32.
  const int fr = lane & 31;
  const int lc = 2 * wave + (lane >> 5);
  int xoff[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i)
    xoff[i] = (i * 32 + fr) * C::BK + swz16(i * 32 + fr, lc) * 16;
  const int woff =
      (C::A_ROWS + fr) * C::BK + swz16(C::A_ROWS + fr, lc) * 16;
  const bool last_half = (halves & 1) != 0;

  v16i acc[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0;

  // Ring: stages 0 .. NS-2 requested up front (a stage past the end
  // reloads the last one, so every step issues the same loads); at stage kt
  // the wave waits for its loads of stage kt, all waves meet (every load of
  // stage kt has landed; every read of stage kt-1 is done), stage
  // kt + NS - 1 goes into stage kt-1's slot, then the wave's k-step.
#pragma unroll
  for (int st = 0; st < C::NS - 1; ++st) issue(st, st);
  for (int kt = 0; kt < nst; ++kt) {
    wait_vmcnt<(C::NS - 2) * C::LOADS>();
    wait_lgkm<0>();
    block_barrier();
    issue((kt + C::NS - 1) % C::NS, kt + C::NS - 1);
    const int8_t *slot = smem + (kt % C::NS) * C::STAGE;
    if (!(last_half && kt == nst - 1 && wave >= 4)) {
      const v4i wf = read_lds16(slot, woff);
      v4i xf[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) xf[i] = read_lds16(slot, xoff[i]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
        acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf, xf[i], acc[i], 0,
                                                       0, 0);
    }
  }
  wait_vmcnt<0>();  // the drain copies have landed before the ring is reused
  wait_lgkm<0>();
  block_barrier();

  // Each wave's sums, [token][channel] in its LDS region: register 4g + t of
  // accumulator i holds token 32 i + (lane mod 32) and channel
  // 8 g + 4 (lane / 32) + t.
  int *red = reinterpret_cast<int *>(smem);
  int *mine = red + wave * C::WAVE;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int m = i * 32 + fr;
      const int c = 8 * g + 4 * (lane >> 5);
      *reinterpret_cast<v4i *>(mine + m * C::ROW + c) =
          v4i{acc[i][4 * g], acc[i][4 * g + 1], acc[i][4 * g + 2],
              acc[i][4 * g + 3]};
    }
  __syncthreads();

  // Four outputs per thread: token m, channels c .. c + 3.
  for (int q = threadIdx.x; q < 32 * TM * 8; q += kSkinnyThreads) {
    const int m = q / 8, c = (q % 8) * 4;
    v4i s = v4i{0, 0, 0, 0};
#pragma unroll
    for (int w = 0; w < kSkinnyWaves; ++w)
      s += *reinterpret_cast<const v4i *>(red + w * C::WAVE + m * C::ROW + c);
    if (m >= p.M) continue;
    const int nn = n0 + c;
    const int64_t o = (int64_t)m * p.N + nn;
    if (EPI == EPI_I32) {
      *reinterpret_cast<v4i *>(static_cast<int *>(p.out) + o) = s;
      continue;
    }
    const float sam = p.sa[m];
    const float4 swn = load_scale4(p.sw, nn, p.vec_sw);
    float t0 = ((float)s.x * sam) * swn.x;
    float t1 = ((float)s.y * sam) * swn.y;
    float t2 = ((float)s.z * sam) * swn.z;
    float t3 = ((float)s.w * sam) * swn.w;
    if (p.bias) {
      const float4 bv = load_bias4(p.bias, nn, p.vec_bias);
      t0 = t0 + bv.x;
      t1 = t1 + bv.y;
      t2 = t2 + bv.z;
      t3 = t3 + bv.w;
    }
    if (EPI == EPI_FP32) {
      *reinterpret_cast<float4 *>(static_cast<float *>(p.out) + o) =
          make_float4(t0, t1, t2, t3);
    } else {
      uint2 v;
      v.x = pack_bf16x2(t0, t1);
      v.y = pack_bf16x2(t2, t3);
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.out) + o) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Tile configurations
// ---------------------------------------------------------------------------
// Large M: 256x256 tiles, 8 waves (two per SIMD) of 64x128, two slots of
// 128-byte K stages (128 KiB LDS): each direct load then fills whole
// 128-byte lines of 8 rows, where 64-byte stages used half lines of 16 rows
// (5% faster on the DiT shapes).  Small M: 64x128 tiles, 4 waves of 64x32,
// 128-byte stages: a 4-slot ring (96 KiB, three stages in flight) when few
// tiles split K, two slots (48 KiB, three work groups per CU) when the
// tiles fill the chip unsplit.
#ifndef W8A8_CFG_LARGE
#define W8A8_CFG_LARGE 256, 256, 128, 4, 2, 4, 2
#endif
#ifndef W8A8_CFG_SKINNY
#define W8A8_CFG_SKINNY 64, 128, 128, 1, 4, 1, 4
#endif
#ifndef W8A8_CFG_MID
#define W8A8_CFG_MID 64, 128, 128, 1, 4, 1, 2
#endif
using CfgLarge = Cfg<W8A8_CFG_LARGE>;
using CfgSkinny = Cfg<W8A8_CFG_SKINNY>;
using CfgMid = Cfg<W8A8_CFG_MID>;

template <class C>
hipError_t set_lds_limit();

template <class C, int EPI>
void launch_main(const KernelArgs &p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_kernel<C, EPI>), grid, dim3(C::THREADS), C::LDS,
                     stream, p);
}

// Dynamic LDS above 64 KiB needs an explicit opt-in: once per device for
// each configuration (the result is kept, errors included).
template <class C>
hipError_t ensure_lds_limit() {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::unordered_map<int, hipError_t> done;
  std::lock_guard<std::mutex> lock(mu);
  const auto it = done.find(dev);
  if (it != done.end()) return it->second;
  const hipError_t r = set_lds_limit<C>();
  done[dev] = r;
  return r;
}

template <class C>
hipError_t launch_cfg(const GemmArgs &g, const GemmPlan &plan,
                      hipStream_t stream) {
  const hipError_t lds_ok = ensure_lds_limit<C>();
  if (lds_ok != hipSuccess) return lds_ok;
  KernelArgs p;
  p.a = g.a;
  p.sa = g.sa;
  p.w = g.w;
  p.sw = g.sw;
  p.bias = g.bias;
  p.M = (int)g.M;
  p.N = (int)g.N;
  p.K = (int)g.K;
  p.tiles_m = (int)((g.M + C::BM - 1) / C::BM);
  p.tiles_n = (int)((g.N + C::BN - 1) / C::BN);
  p.stages_total = (int)(g.K / C::BK);
  p.splits = plan.splits;
  p.group_m = plan.group_m;
  p.tile_base = 0;
  p.remap = 1;
  const bool vb_sw = (reinterpret_cast<uintptr_t>(g.sw) & 15) == 0;
  const bool vb_bias = (reinterpret_cast<uintptr_t>(g.bias) & 7) == 0;
  p.vec_sw = vb_sw;
  p.vec_bias = vb_bias;
  const dim3 grid((unsigned)plan.main_tiles, 1, (unsigned)plan.splits);
  if (plan.splits == 1) {
    p.out = g.out;
    switch (g.epi) {
      case EPI_BF16: launch_main<C, EPI_BF16>(p, grid, stream); break;
      case EPI_FP32: launch_main<C, EPI_FP32>(p, grid, stream); break;
      default: launch_main<C, EPI_I32>(p, grid, stream); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.tail_splits <= 1) return e;
    // Tail: the last tiles (less than one wave of the chip) split K so the
    // chip stays busy; INT32 slices in the workspace, then a reduction.
    KernelArgs t = p;
    t.out = g.workspace;
    t.splits = plan.tail_splits;
    t.tile_base = plan.main_tiles;
    t.remap = 0;
    launch_main<C, EPI_PARTIAL_TILE>(
        t, dim3((unsigned)plan.tail_tiles, 1, (unsigned)plan.tail_splits),
        stream);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int QB = C::BM * C::BN / 4 / 256;
    const dim3 rgrid((unsigned)(plan.tail_tiles * QB));
    const int *part = static_cast<const int *>(g.workspace);
#define W8A8_TAIL(E)                                                          \
  hipLaunchKernelGGL((tail_reduce_kernel<C, E>), rgrid, dim3(256),           \
                     0, stream, part, plan.tail_splits, plan.tail_tiles,     \
                     plan.main_tiles, p.tiles_m, p.tiles_n, p.group_m, g.sa, \
                     g.sw, g.bias, g.out, p.M, p.N, vb_sw, vb_bias)
    switch (g.epi) {
      case EPI_BF16: W8A8_TAIL(EPI_BF16); break;
      case EPI_FP32: W8A8_TAIL(EPI_FP32); break;
      default: W8A8_TAIL(EPI_I32); break;
    }
#undef W8A8_TAIL
    return hipGetLastError();
  }
  p.out = g.workspace;
  launch_main<C, EPI_PARTIAL>(p, grid, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t quads = g.M * g.N / 4;
  int64_t blocks = (quads + 255) / 256;
  if (blocks > 256 * 8) blocks = 256 * 8;
  const int *part = static_cast<const int *>(g.workspace);
  switch (g.epi) {
    case EPI_BF16:
      hipLaunchKernelGGL(splitk_reduce_kernel<EPI_BF16>, dim3((unsigned)blocks),
                         dim3(256), 0, stream, part, plan.splits, g.sa, g.sw,
                         g.bias, g.out, p.M, p.N, vb_sw, vb_bias);
      break;
    case EPI_FP32:
      hipLaunchKernelGGL(splitk_reduce_kernel<EPI_FP32>, dim3((unsigned)blocks),
                         dim3(256), 0, stream, part, plan.splits, g.sa, g.sw,
                         g.bias, g.out, p.M, p.N, vb_sw, vb_bias);
      break;
    default:
      hipLaunchKernelGGL(splitk_reduce_kernel<EPI_I32>, dim3((unsigned)blocks),
                         dim3(256), 0, stream, part, plan.splits, g.sa, g.sw,
                         g.bias, g.out, p.M, p.N, vb_sw, vb_bias);
      break;
  }
  return hipGetLastError();
}

template <class C>
hipError_t set_lds_limit() {
  // Opt in to more than 64 KiB of dynamic LDS where a configuration needs it.
  hipError_t e = hipSuccess;
  if (C::LDS > 64 * 1024) {
    e = hipFuncSetAttribute((const void *)gemm_kernel<C, EPI_BF16>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void *)gemm_kernel<C, EPI_FP32>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void *)gemm_kernel<C, EPI_I32>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void *)gemm_kernel<C, EPI_PARTIAL>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void *)gemm_kernel<C, EPI_PARTIAL_TILE>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
  }
  return e;
}

constexpr int kCfgLarge = 0;
constexpr int kCfgSkinny = 1;
constexpr int kCfgMid = 2;
constexpr int kCfgSingle = 3;  // skinny_kernel: at most 64 tokens, one launch
constexpr int kCUs = 256;

template <int TM>
hipError_t set_skinny_lds() {
  hipError_t e = hipSuccess;
  constexpr int lds = SkinnyCfg<TM>::LDS;
  if (lds > 64 * 1024) {
    e = hipFuncSetAttribute((const void *)skinny_kernel<TM, EPI_BF16>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void *)skinny_kernel<TM, EPI_FP32>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void *)skinny_kernel<TM, EPI_I32>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  }
  return e;
}

// Dynamic LDS above 64 KiB, opted in once per device (result kept).
template <int TM>
hipError_t ensure_skinny_lds() {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::unordered_map<int, hipError_t> done;
  std::lock_guard<std::mutex> lock(mu);
  const auto it = done.find(dev);
  if (it != done.end()) return it->second;
  const hipError_t r = set_skinny_lds<TM>();
  done[dev] = r;
  return r;
}

template <int TM>
hipError_t launch_skinny(const GemmArgs &g, hipStream_t stream) {
  const hipError_t lds_ok = ensure_skinny_lds<TM>();
  if (lds_ok != hipSuccess) return lds_ok;
  KernelArgs p{};
  p.a = g.a;
  p.sa = g.sa;
  p.w = g.w;
  p.sw = g.sw;
  p.bias = g.bias;
  p.out = g.out;
  p.M = (int)g.M;
  p.N = (int)g.N;
  p.K = (int)g.K;
  p.vec_sw = (reinterpret_cast<uintptr_t>(g.sw) & 15) == 0;
  p.vec_bias = (reinterpret_cast<uintptr_t>(g.bias) & 7) == 0;
  const dim3 grid((unsigned)(g.N / 32));
  constexpr int lds = SkinnyCfg<TM>::LDS;
  switch (g.epi) {
    case EPI_BF16:
      hipLaunchKernelGGL((skinny_kernel<TM, EPI_BF16>), grid,
                         dim3(kSkinnyThreads), lds, stream, p);
      break;
    case EPI_FP32:
      hipLaunchKernelGGL((skinny_kernel<TM, EPI_FP32>), grid,
                         dim3(kSkinnyThreads), lds, stream, p);
      break;
    default:
      hipLaunchKernelGGL((skinny_kernel<TM, EPI_I32>), grid,
                         dim3(kSkinnyThreads), lds, stream, p);
      break;
  }
  return hipGetLastError();
}

// Token tiles per group of the tile order: a narrow output (few channel
// tiles) affords taller groups within one wave of work groups.
#ifndef W8A8_GROUP_M_NARROW
#define W8A8_GROUP_M_NARROW 4
#endif
#ifndef W8A8_GROUP_M_WIDE
#define W8A8_GROUP_M_WIDE 4
#endif
#ifndef W8A8_SKINNY_WGS_PER_CU
#define W8A8_SKINNY_WGS_PER_CU 1
#endif
#ifndef W8A8_SKINNY_MIN_STAGES
#define W8A8_SKINNY_MIN_STAGES 4
#endif
// Fewest K slices that make a split tail launch worthwhile, and the least
// K (bytes) of one slice.
#ifndef W8A8_TAIL_MIN_SPLITS
#define W8A8_TAIL_MIN_SPLITS 2
#endif
#ifndef W8A8_TAIL_MIN_K
#define W8A8_TAIL_MIN_K 512
#endif
// Fewer than a wave of 256x256 tiles still runs as one partial wave of
// them when the 64x128 tiles would not all be resident at once (three work
// groups per CU) or when there are at least this many large tiles: one
// large-tile time then beats the small tiles (measured at N=5376, K=5376:
// M=1280, 105 large tiles, 61 us against 81 us of small tiles; M=1024, 84
// large tiles, small tiles win with 55 us).
#ifndef W8A8_SINGLE_MAX_N
#define W8A8_SINGLE_MAX_N 16384
#endif
#ifndef W8A8_SINGLE_MAX_K
#define W8A8_SINGLE_MAX_K 16384
#endif
#ifndef W8A8_LARGE_MIN_TILES
#define W8A8_LARGE_MIN_TILES 112
#endif

}  // namespace

// Scratch of w8a8_gemm_noalloc (callers that cannot allocate device
// memory): the INT32 partial sums of the split-K launches live here instead
// of in a caller's workspace.  The planner never needs more than 64 MiB of
// partials: a split tail has fewer than 256 tiles, and tiles x slices stays
// at or below 256 slices of one 256 x 256 INT32 tile (256 KiB each); the
// skinny split-K plans at most 256 / tiles slices of an M x N tile grid of
// 64 x 128 tiles, at most 8 MiB.  Host code never passes the array's name
// to a kernel (in host code it is a stand-in, not a device address): it
// uses the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
std::unordered_map<int, void *> g_scratch_addr;
}  // namespace

hipError_t resolve_scratch(int device) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr.count(device)) return hipSuccess;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != device) return hipErrorInvalidDevice;
  void *ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (ptr == nullptr) return hipErrorInvalidSymbol;
  g_scratch_addr[device] = ptr;
  return hipSuccess;
}

void *scratch_on_device(int device) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  const auto it = g_scratch_addr.find(device);
  return it == g_scratch_addr.end() ? nullptr : it->second;
}

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K) {
  GemmPlan plan{kCfgLarge, 1, CfgLarge::GROUP_M, 0, 0, 0, 0, 0};
  // At most 64 tokens: one launch, no partial sums (skinny_kernel), while
  // its N / 32 work groups stay within two per CU and K within 16384
  // (measured at M = 64, against the split-K tiles below: N = K = 5376
  // 7.9 against 12.0 us, N = 16128 19.1 against 20.0 us; N = 21504 25.8
  // against 19.7 us, K = 21504 25.2 against 24.4 us).
  if (M <= 64 && N <= W8A8_SINGLE_MAX_N && K <= W8A8_SINGLE_MAX_K) {
    plan.config = kCfgSingle;
    plan.skinny_tm = M <= 32 ? 1 : 2;
    plan.main_tiles = (int)(N / 32);
    return plan;
  }
  const int64_t tiles_n = (N + CfgLarge::BN - 1) / CfgLarge::BN;
  plan.group_m = tiles_n <= 32 ? W8A8_GROUP_M_NARROW : W8A8_GROUP_M_WIDE;
  const int64_t large_tiles = ((M + CfgLarge::BM - 1) / CfgLarge::BM) * tiles_n;
  if (large_tiles >= kCUs) {
    plan.main_tiles = (int)large_tiles;
    // A last partial wave of tiles leaves most CUs idle for a whole tile
    // time.  When it holds few tiles, run it as a second launch whose tiles
    // split K so that about one wave of work groups shares it (each slice
    // keeps at least W8A8_TAIL_MIN_K bytes of K).
    const int64_t rem = large_tiles % kCUs;
    const int64_t stages = K / CfgLarge::BK;
    const int64_t splits = std::min<int64_t>(
        rem ? kCUs / rem : 0, stages / (W8A8_TAIL_MIN_K / CfgLarge::BK));
    if (rem > 0 && splits >= W8A8_TAIL_MIN_SPLITS) {
      plan.main_tiles = (int)(large_tiles - rem);
      plan.tail_tiles = (int)rem;
      plan.tail_splits = (int)splits;
      plan.workspace = (size_t)(rem * splits) * CfgLarge::BM * CfgLarge::BN *
                       sizeof(int32_t);
    }
    return plan;
  }
  const int64_t tiles =
      ((M + CfgSkinny::BM - 1) / CfgSkinny::BM) * ((N + CfgSkinny::BN - 1) / CfgSkinny::BN);
  constexpr int64_t kMidResident = (160 * 1024 / CfgMid::LDS) * kCUs;
  if (large_tiles >= W8A8_LARGE_MIN_TILES || tiles > kMidResident) {
    plan.main_tiles = (int)large_tiles;
    return plan;
  }
  // Few tiles: smaller tiles, and split K so that about
  // W8A8_SKINNY_WGS_PER_CU work groups per CU stream the weights, each
  // slice keeping at least W8A8_SKINNY_MIN_STAGES stages.
  plan.config = kCfgSkinny;
  plan.group_m = CfgSkinny::GROUP_M;
  plan.main_tiles = (int)tiles;
  const int64_t stages = K / CfgSkinny::BK;
  const int64_t splits = std::max<int64_t>(
      1, std::min<int64_t>(kCUs * W8A8_SKINNY_WGS_PER_CU / tiles,
                           stages / W8A8_SKINNY_MIN_STAGES));
  plan.splits = (int)splits;
  plan.workspace = splits > 1 ? (size_t)(splits * M * N * sizeof(int32_t)) : 0;
  // A wave or more of small tiles: no split, and 128-byte stages.
  if (splits == 1 && tiles >= kCUs) {
    static_assert(CfgMid::BM == CfgSkinny::BM && CfgMid::BN == CfgSkinny::BN,
                  "same tiles");
    plan.config = kCfgMid;
  }
  return plan;
}

bool plan_launchable(const GemmPlan &plan) {
  // A launch holds fewer than 2^32 work-items per grid dimension.
  const uint64_t lim = 0xFFFFFFFFull;
  const uint64_t threads = plan.config == kCfgLarge    ? CfgLarge::THREADS
                           : plan.config == kCfgMid    ? CfgMid::THREADS
                           : plan.config == kCfgSingle ? kSkinnyThreads
                                                       : CfgSkinny::THREADS;
  if ((uint64_t)plan.main_tiles * threads > lim) return false;
  if ((uint64_t)plan.tail_tiles * threads > lim) return false;
  return (uint64_t)plan.tail_tiles * (CfgLarge::BM * CfgLarge::BN / 4) <= lim;
}

hipError_t launch_gemm(const GemmArgs &args, const GemmPlan &plan,
                       hipStream_t stream) {
  // The partial sums of a split plan go to the workspace: refuse to launch
  // without one of the planned size (the API layer checks this first; this
  // guards direct callers of the launcher).
  if (plan.workspace > 0 &&
      (args.workspace == nullptr || args.workspace_bytes < plan.workspace))
    return hipErrorInvalidValue;
  if (plan.config == kCfgLarge) return launch_cfg<CfgLarge>(args, plan, stream);
  if (plan.config == kCfgMid) return launch_cfg<CfgMid>(args, plan, stream);
  if (plan.config == kCfgSingle)
    return plan.skinny_tm == 1 ? launch_skinny<1>(args, stream)
                               : launch_skinny<2>(args, stream);
  return launch_cfg<CfgSkinny>(args, plan, stream);
}

}  // namespace w8a8

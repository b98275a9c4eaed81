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
//     LDS, double buffered.  Tiles are filled with global_load_lds_dwordx4
//     (direct global -> LDS, 16 bytes per lane), so staging costs no VGPRs.
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

#pragma clang fp contract(off)

namespace w8a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void gbl_void;

constexpr int kXcds = 8;
constexpr int EPI_PARTIAL = 3;  // split-K slice: raw INT32 to the workspace

template <int BM_, int BN_, int BK_, int WGM_, int WGN_, int GROUP_M_>
struct Cfg {
  static constexpr int BM = BM_;   // tokens per block tile
  static constexpr int BN = BN_;   // output channels per block tile
  static constexpr int BK = BK_;   // K bytes per LDS stage
  static constexpr int WGM = WGM_; // waves along M
  static constexpr int WGN = WGN_; // waves along N
  static constexpr int GROUP_M = GROUP_M_;
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
  static constexpr int LDS = 2 * STAGE;
  static constexpr int A_LOADS = A_BYTES / (1024 * WAVES);  // per wave
  static constexpr int B_LOADS = B_BYTES / (1024 * WAVES);
  static_assert(BK == 64 || BK == 128, "BK");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile");
  static_assert(A_BYTES % (1024 * WAVES) == 0, "A staging");
  static_assert(B_BYTES % (1024 * WAVES) == 0, "B staging");
  static_assert(LDS <= 160 * 1024, "LDS");
};

// Position of logical 16-byte chunk c in LDS row r (an involution in c).
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  if (CPR == 4) return c ^ (((r >> 1) ^ (r >> 3)) & 3);
  return c ^ (((r >> 1) ^ ((r & 1) << 2)) & 7);
}

__device__ __forceinline__ void load_lds16(const int8_t *g, lds_void *l) {
  __builtin_amdgcn_global_load_lds((gbl_void *)g, l, 16, 0, 0);
}

__device__ __forceinline__ v4i read_lds16(const int8_t *lds_base, int off) {
  return *reinterpret_cast<const v4i *>(lds_base + off);
}

// Block id -> (token tile, channel tile).
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n,
                                        int group_m, int &tm, int &tn) {
  const int T = tiles_m * tiles_n;
  const int xcd = bid % kXcds;
  const int local = bid / kXcds;
  const int per = T / kXcds, rem = T % kXcds;
  const int L = xcd * per + min(xcd, rem) + local;
  const int span = group_m * tiles_n;
  const int g = L / span;
  const int first = g * group_m;
  const int gsize = min(tiles_m - first, group_m);
  const int within = L - g * span;
  tm = first + within % gsize;
  tn = within / gsize;
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
  tile_of(blockIdx.x, p.tiles_m, p.tiles_n, C::GROUP_M, tm, tn);
  const int m0 = tm * C::BM;
  const int n0 = tn * C::BN;

  // K stages of this split.
  const int z = blockIdx.z;
  const int kt0 = (int)((int64_t)z * p.stages_total / p.splits);
  const int kt1 = (int)((int64_t)(z + 1) * p.stages_total / p.splits);
  const int nk = kt1 - kt0;

  // Per-lane global source of each direct load (stage 0 of this split).
  const int8_t *ga[C::A_LOADS];
  const int8_t *gb[C::B_LOADS];
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) {
    const int slot = (j * C::WAVES + wave) * 64 + lane;
    const int r = slot / C::CPR;
    const int c = swz<C::CPR>(r, slot % C::CPR);
    const int row = min(m0 + r, p.M - 1);
    ga[j] = p.a + (int64_t)row * p.K + (int64_t)kt0 * C::BK + c * 16;
  }
#pragma unroll
  for (int j = 0; j < C::B_LOADS; ++j) {
    const int slot = (j * C::WAVES + wave) * 64 + lane;
    const int r = slot / C::CPR;
    const int c = swz<C::CPR>(r, slot % C::CPR);
    const int row = min(n0 + r, p.N - 1);
    gb[j] = p.w + (int64_t)row * p.K + (int64_t)kt0 * C::BK + c * 16;
  }

  auto issue = [&](int stage_idx, int buf) {
    int8_t *sa_base = smem + buf * C::STAGE;
    int8_t *sb_base = sa_base + C::A_BYTES;
    const int64_t koff = (int64_t)stage_idx * C::BK;
#pragma unroll
    for (int j = 0; j < C::A_LOADS; ++j)
      load_lds16(ga[j] + koff,
                 (lds_void *)(sa_base + (j * C::WAVES + wave) * 1024));
#pragma unroll
    for (int j = 0; j < C::B_LOADS; ++j)
      load_lds16(gb[j] + koff,
                 (lds_void *)(sb_base + (j * C::WAVES + wave) * 1024));
  };

  // Fragment read offsets (bytes within a tile) for k-step 0; the k-step
  // adds 2 chunks, which the swizzle maps with a per-row XOR.
  const int frow = lane & 31;
  const int fchunk = lane >> 5;

  v16i acc[C::TN][C::TM];
#pragma unroll
  for (int i = 0; i < C::TN; ++i)
#pragma unroll
    for (int j = 0; j < C::TM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  if (nk > 0) issue(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 1 < nk) issue(kt + 1, (kt + 1) & 1);
    const int8_t *sa_base = smem + (kt & 1) * C::STAGE;
    const int8_t *sb_base = sa_base + C::A_BYTES;
#pragma unroll
    for (int ks = 0; ks < C::BK / 32; ++ks) {
      v4i xa[C::TM], wb[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        const int r = wave_m * C::WM + i * 32 + frow;
        xa[i] = read_lds16(sa_base,
                           r * C::BK + swz<C::CPR>(r, ks * 2 + fchunk) * 16);
      }
#pragma unroll
      for (int i = 0; i < C::TN; ++i) {
        const int r = wave_n * C::WN + i * 32 + frow;
        wb[i] = read_lds16(sb_base,
                           r * C::BK + swz<C::CPR>(r, ks * 2 + fchunk) * 16);
      }
#pragma unroll
      for (int i = 0; i < C::TN; ++i)
#pragma unroll
        for (int j = 0; j < C::TM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wb[i], xa[j],
                                                            acc[i][j], 0, 0, 0);
    }
  }

  // Epilogue.  Lane holds token m = base + (lane & 31) and, for register
  // 4g + t, channel n = base + 8g + 4*(lane >> 5) + t.
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
        const float4 swn = *reinterpret_cast<const float4 *>(p.sw + n);
        float t0 = ((float)acc0 * sam) * swn.x;
        float t1 = ((float)acc1 * sam) * swn.y;
        float t2 = ((float)acc2 * sam) * swn.z;
        float t3 = ((float)acc3 * sam) * swn.w;
        if (p.bias) {
          const uint2 b = *reinterpret_cast<const uint2 *>(p.bias + n);
          t0 = t0 + bf16_to_f32(b.x & 0xFFFFu);
          t1 = t1 + bf16_to_f32(b.x >> 16);
          t2 = t2 + bf16_to_f32(b.y & 0xFFFFu);
          t3 = t3 + bf16_to_f32(b.y >> 16);
        }
        if (EPI == EPI_FP32) {
          *reinterpret_cast<float4 *>(static_cast<float *>(p.out) + o) =
              make_float4(t0, t1, t2, t3);
        } else {
          uint2 v;
          v.x = f32_to_bf16_rne(t0) | (f32_to_bf16_rne(t1) << 16);
          v.y = f32_to_bf16_rne(t2) | (f32_to_bf16_rne(t3) << 16);
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
    void *__restrict__ out, int M, int N) {
  const int64_t MN = (int64_t)M * N;
  const int64_t quads = MN / 4;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < quads;
       q += (int64_t)gridDim.x * 256) {
    const int64_t o = q * 4;
    v4i s = *reinterpret_cast<const v4i *>(part + o);
    for (int z = 1; z < splits; ++z)
      s += *reinterpret_cast<const v4i *>(part + z * MN + o);
    if (EPI == EPI_I32) {
      *reinterpret_cast<v4i *>(static_cast<int *>(out) + o) = s;
      continue;
    }
    const int m = (int)(o / N);
    const int n = (int)(o - (int64_t)m * N);
    const float sam = sa[m];
    const float4 swn = *reinterpret_cast<const float4 *>(sw + n);
    float t0 = ((float)s.x * sam) * swn.x;
    float t1 = ((float)s.y * sam) * swn.y;
    float t2 = ((float)s.z * sam) * swn.z;
    float t3 = ((float)s.w * sam) * swn.w;
    if (bias) {
      const uint2 b = *reinterpret_cast<const uint2 *>(bias + n);
      t0 = t0 + bf16_to_f32(b.x & 0xFFFFu);
      t1 = t1 + bf16_to_f32(b.x >> 16);
      t2 = t2 + bf16_to_f32(b.y & 0xFFFFu);
      t3 = t3 + bf16_to_f32(b.y >> 16);
    }
    if (EPI == EPI_FP32) {
      *reinterpret_cast<float4 *>(static_cast<float *>(out) + o) =
          make_float4(t0, t1, t2, t3);
    } else {
      uint2 v;
      v.x = f32_to_bf16_rne(t0) | (f32_to_bf16_rne(t1) << 16);
      v.y = f32_to_bf16_rne(t2) | (f32_to_bf16_rne(t3) << 16);
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + o) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Tile configurations
// ---------------------------------------------------------------------------
using CfgLarge = Cfg<256, 256, 64, 2, 2, 8>;   // large M: 4 waves, 128x128 each
using CfgSkinny = Cfg<64, 128, 64, 1, 4, 1>;   // small M: 4 waves, 64x32 each

template <class C>
hipError_t launch_cfg(const GemmArgs &g, int splits, hipStream_t stream) {
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
  p.splits = splits;
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n), 1, (unsigned)splits);
  const dim3 block(C::THREADS);
  if (splits == 1) {
    p.out = g.out;
    switch (g.epi) {
      case EPI_BF16:
        hipLaunchKernelGGL((gemm_kernel<C, EPI_BF16>), grid, block, C::LDS,
                           stream, p);
        break;
      case EPI_FP32:
        hipLaunchKernelGGL((gemm_kernel<C, EPI_FP32>), grid, block, C::LDS,
                           stream, p);
        break;
      default:
        hipLaunchKernelGGL((gemm_kernel<C, EPI_I32>), grid, block, C::LDS,
                           stream, p);
        break;
    }
    return hipGetLastError();
  }
  p.out = g.workspace;
  hipLaunchKernelGGL((gemm_kernel<C, EPI_PARTIAL>), grid, block, C::LDS,
                     stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t quads = g.M * g.N / 4;
  int64_t blocks = (quads + 255) / 256;
  if (blocks > 256 * 8) blocks = 256 * 8;
  const int *part = static_cast<const int *>(g.workspace);
  switch (g.epi) {
    case EPI_BF16:
      hipLaunchKernelGGL(splitk_reduce_kernel<EPI_BF16>, dim3((unsigned)blocks),
                         dim3(256), 0, stream, part, splits, g.sa, g.sw,
                         g.bias, g.out, p.M, p.N);
      break;
    case EPI_FP32:
      hipLaunchKernelGGL(splitk_reduce_kernel<EPI_FP32>, dim3((unsigned)blocks),
                         dim3(256), 0, stream, part, splits, g.sa, g.sw,
                         g.bias, g.out, p.M, p.N);
      break;
    default:
      hipLaunchKernelGGL(splitk_reduce_kernel<EPI_I32>, dim3((unsigned)blocks),
                         dim3(256), 0, stream, part, splits, g.sa, g.sw,
                         g.bias, g.out, p.M, p.N);
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
  }
  return e;
}

constexpr int kCfgLarge = 0;
constexpr int kCfgSkinny = 1;
constexpr int kCUs = 256;

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K) {
  GemmPlan plan{kCfgLarge, 1, 0};
  const int64_t large_tiles =
      ((M + CfgLarge::BM - 1) / CfgLarge::BM) * ((N + CfgLarge::BN - 1) / CfgLarge::BN);
  if (large_tiles >= kCUs) return plan;
  // Few tiles: smaller tiles, and split K while the grid is under one wave
  // of the chip and each slice keeps at least 8 stages.
  plan.config = kCfgSkinny;
  const int64_t tiles =
      ((M + CfgSkinny::BM - 1) / CfgSkinny::BM) * ((N + CfgSkinny::BN - 1) / CfgSkinny::BN);
  const int64_t stages = K / CfgSkinny::BK;
  int splits = 1;
  while (tiles * splits * 2 <= kCUs && stages / (splits * 2) >= 8) splits *= 2;
  plan.splits = splits;
  plan.workspace = splits > 1 ? (size_t)(splits * M * N * sizeof(int32_t)) : 0;
  return plan;
}

hipError_t launch_gemm(const GemmArgs &args, const GemmPlan &plan,
                       hipStream_t stream) {
  if (plan.config == kCfgLarge) return launch_cfg<CfgLarge>(args, plan.splits, stream);
  return launch_cfg<CfgSkinny>(args, plan.splits, stream);
}

}  // namespace w8a8

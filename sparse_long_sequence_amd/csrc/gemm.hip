// Encoder-layer GEMMs on the gfx950 matrix cores, with fused epilogues, and the
// LayerNorm row kernel.
//
// [FT-LF] = the page "FasterTransformer Longformer 推理加速实践：PyTorch 集成、输入约束与
// 端到端性能解析", section "Longformer Encoder 计算流程", per-layer steps:
//   1  the Q / K / V / global-K / global-V projections (one packed GEMM) and the
//      global-query projection of the leading G tokens, bias added and the result
//      split into heads;                                  -> epilogue kEpiHeads
//   5  attention output projection + bias + residual, then LayerNorm
//                                                         -> kEpiResidT + layernorm
//   6  FFN: GEMM + bias + GELU, GEMM + bias + residual, then LayerNorm
//                                                         -> kEpiGelu, kEpiResidF32
// (steps 3-4, the attention itself, are attn_mfma.hip).
//
// C[m, n] = sum_k A[arow(m), k] * W[n, k] + bias[n]: both operands are read as rows
// of consecutive k, which is the operand layout of v_mfma_f32_32x32x16 (lane (n, g)
// holds 8 consecutive k of one row).  The weight rows are the MFMA's first operand
// and the activation rows its second, so each lane's 16 accumulators are 4 groups
// of 4 consecutive output columns of ONE output row: the epilogue stores 8-byte
// runs.  Workgroup tile 128 x 128, K step 64, 4 waves each owning 64 x 64 (2 x 2
// MFMA tiles); operands staged through double-buffered LDS (pitch 144 B: the
// 16-byte fragment reads are conflict-free); the next K step's global loads are in
// flight while the current one is multiplied.  Rows of A past M read out of range
// (zeros) and are not stored.
#include "lf_device.h"
#include "lf_internal.h"

namespace lf {

namespace {

constexpr int kGT = 128;      // tile rows and columns
constexpr int kGK = 64;       // K step
constexpr int kGld = 72;      // LDS row pitch (elements)
constexpr int kGThreads = 256;
constexpr int kGroupM = 8;    // m-tiles per group of the tile order (L2 reuse of W tiles)

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ inline rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// The erf form of GELU ([FT-LF] step 6 names GELU; the exact form is the reading).
__device__ inline float gelu(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

template <typename T, int EPI>
__global__ __launch_bounds__(kGThreads) void gemm_kernel(GemmArgs g) {
  typedef typename Elem<T>::vec8 v8;
  typedef typename Elem<T>::vec4 v4;
  __shared__ __attribute__((aligned(16))) T sa[2][kGT * kGld];
  __shared__ __attribute__((aligned(16))) T sw[2][kGT * kGld];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int n = lane & 31, gq = lane >> 5;

  // tile order: groups of kGroupM m-tiles sweep all n-tiles, so a W tile is reused
  // by neighbouring workgroups while it is in L2
  const int tiles_n = g.N / kGT;
  const int tiles_m = (g.M + kGT - 1) / kGT;
  const int bid = blockIdx.x;
  const int per_group = kGroupM * tiles_n;
  const int grp = bid / per_group;
  const int first_m = grp * kGroupM;
  const int gsize = min(kGroupM, tiles_m - first_m);
  const int in_grp = bid - grp * per_group;
  const int tm = __builtin_amdgcn_readfirstlane(first_m + in_grp % gsize);
  const int tn = __builtin_amdgcn_readfirstlane(in_grp / gsize);
  const int m0 = tm * kGT, n0 = tn * kGT;

  // global -> register mapping: thread t loads 16 B at column 8 (t % 8) of rows
  // t / 8 + 32 i (i = 0..3) of both tiles
  const int lr = t >> 3, lc = 8 * (t & 7);
  const rsrc_t ra = make_rsrc(g.a, 0x7fffffff);
  const rsrc_t rw = make_rsrc(g.w, 0x7fffffff);
  int aoff[4], woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + lr + 32 * i;
    const int arow = g.a_group > 0 ? (m / g.a_group) * g.a_group_stride + m % g.a_group : m;
    aoff[i] = m < g.M ? (arow * g.lda + lc) * (int)sizeof(T) : -1;
    woff[i] = ((n0 + lr + 32 * i) * g.ldw + lc) * (int)sizeof(T);
  }
  u32x4 pa[4], pw[4];
  auto load = [&](int ks) {
    const int kb = ks * kGK * (int)sizeof(T);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pa[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, aoff[i] < 0 ? -1 : aoff[i] + kb, 0, 0);
      pw[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, woff[i] + kb, 0, 0);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(u32x4*)&sa[buf][(lr + 32 * i) * kGld + lc] = pa[i];
      *(u32x4*)&sw[buf][(lr + 32 * i) * kGld + lc] = pw[i];
    }
  };

  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  f32x16 acc[2][2];   // [n sub-tile][m sub-tile]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = g.K / kGK;
  load(0);
  store(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    if (ks + 1 < nk) load(ks + 1);
    const int buf = ks & 1;
#pragma unroll
    for (int kk = 0; kk < kGK / 16; ++kk) {
      v8 wf[2], xf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        wf[i] = *(const v8*)&sw[buf][(wn + 32 * i + n) * kGld + 16 * kk + 8 * gq];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        xf[j] = *(const v8*)&sa[buf][(wm + 32 * j + n) * kGld + 16 * kk + 8 * gq];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(wf[i], xf[j], acc[i][j]);
    }
    if (ks + 1 < nk) store((ks + 1) & 1);
    __syncthreads();
  }

  // epilogue: lane holds, for output row m, columns nb .. nb + 3 of each group
  const T* bias = (const T*)g.bias;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = m0 + wm + 32 * j + n;
    if (m >= g.M) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int nb = n0 + wn + 32 * i + 8 * jj + 4 * gq;
        const v4 bv = *(const v4*)(bias + nb);
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = acc[i][j][4 * jj + e] + Elem<T>::to_f(bv[e]);
        if (EPI == kEpiHeads) {
          // n -> tensor n / D, head (n % D) / 64, dim n % 64; m -> (batch, row)
          const int ti = nb / g.D, nn = nb - ti * g.D;
          const int h = nn >> 6, d = nn & 63;
          const int bb = m / g.rows, rr = m - bb * g.rows;
          T* dst = (T*)g.heads[ti] + (((size_t)bb * g.H + h) * g.rows + rr) * 64 + d;
          v4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = Elem<T>::from_f(r[e]);
          *(v4*)dst = w;
        } else if (EPI == kEpiGelu) {
          v4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = Elem<T>::from_f(gelu(r[e]));
          *(v4*)((T*)g.out + (size_t)m * g.ldo + nb) = w;
        } else {
          f32x4 z;
          if (EPI == kEpiResidF32) {
            const f32x4 rv = *(const f32x4*)((const float*)g.resid + (size_t)m * g.ldr + nb);
#pragma unroll
            for (int e = 0; e < 4; ++e) z[e] = r[e] + rv[e];
          } else {
            const v4 rv = *(const v4*)((const T*)g.resid + (size_t)m * g.ldr + nb);
#pragma unroll
            for (int e = 0; e < 4; ++e) z[e] = r[e] + Elem<T>::to_f(rv[e]);
          }
          *(f32x4*)((float*)g.out + (size_t)m * g.ldo + nb) = z;
        }
      }
    }
  }
}

// LayerNorm of one row per wave ([FT-LF] steps 5 and 6): mean, biased variance
// (two passes over the row held in registers), (z - mean) / sqrt(var + eps) * gamma
// + beta; written as fp32 (the residual stream) and / or in the layer dtype.
template <typename T, int NPL>
__global__ __launch_bounds__(256) void layernorm_kernel(const float* __restrict__ z,
                                                        const T* __restrict__ gamma,
                                                        const T* __restrict__ beta, float eps,
                                                        int M, int N, float* __restrict__ out_f32,
                                                        T* __restrict__ out_t) {
  typedef typename Elem<T>::vec4 v4;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const float* zr = z + (size_t)row * N;
  f32x4 x[NPL];
#pragma unroll
  for (int c = 0; c < NPL; ++c) x[c] = *(const f32x4*)(zr + 4 * (lane + 64 * c));
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < NPL; ++c) s += (x[c][0] + x[c][1]) + (x[c][2] + x[c][3]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
  const float mean = s / (float)N;
  float q = 0.0f;
#pragma unroll
  for (int c = 0; c < NPL; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float dv = x[c][e] - mean;
      q += dv * dv;
    }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) q += __shfl_xor(q, d, 64);
  const float inv = 1.0f / sqrtf(q / (float)N + eps);
#pragma unroll
  for (int c = 0; c < NPL; ++c) {
    const int col = 4 * (lane + 64 * c);
    const v4 gv = *(const v4*)(gamma + col);
    const v4 bv = *(const v4*)(beta + col);
    f32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      y[e] = (x[c][e] - mean) * inv * Elem<T>::to_f(gv[e]) + Elem<T>::to_f(bv[e]);
    if (out_f32) *(f32x4*)(out_f32 + (size_t)row * N + col) = y;
    if (out_t) {
      v4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = Elem<T>::from_f(y[e]);
      *(v4*)(out_t + (size_t)row * N + col) = w;
    }
  }
}

template <typename T>
hipError_t gemm_t(const GemmArgs& g, hipStream_t st) {
  const int tiles = ((g.M + kGT - 1) / kGT) * (g.N / kGT);
  switch (g.epi) {
    case kEpiHeads: gemm_kernel<T, kEpiHeads><<<tiles, kGThreads, 0, st>>>(g); break;
    case kEpiGelu: gemm_kernel<T, kEpiGelu><<<tiles, kGThreads, 0, st>>>(g); break;
    case kEpiResidT: gemm_kernel<T, kEpiResidT><<<tiles, kGThreads, 0, st>>>(g); break;
    case kEpiResidF32: gemm_kernel<T, kEpiResidF32><<<tiles, kGThreads, 0, st>>>(g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t layernorm_t(const float* z, const void* gamma, const void* beta, float eps, int M,
                       int N, float* out_f32, void* out_t, hipStream_t st) {
  const int grid = (M + 3) / 4;
  const T* gm = (const T*)gamma;
  const T* bt = (const T*)beta;
  switch (N / 256) {
    case 1: layernorm_kernel<T, 1><<<grid, 256, 0, st>>>(z, gm, bt, eps, M, N, out_f32, (T*)out_t); break;
    case 2: layernorm_kernel<T, 2><<<grid, 256, 0, st>>>(z, gm, bt, eps, M, N, out_f32, (T*)out_t); break;
    case 3: layernorm_kernel<T, 3><<<grid, 256, 0, st>>>(z, gm, bt, eps, M, N, out_f32, (T*)out_t); break;
    case 4: layernorm_kernel<T, 4><<<grid, 256, 0, st>>>(z, gm, bt, eps, M, N, out_f32, (T*)out_t); break;
    case 8: layernorm_kernel<T, 8><<<grid, 256, 0, st>>>(z, gm, bt, eps, M, N, out_f32, (T*)out_t); break;
    case 16: layernorm_kernel<T, 16><<<grid, 256, 0, st>>>(z, gm, bt, eps, M, N, out_f32, (T*)out_t); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool gemm_shape_ok(int M, int N, int K) {
  return M >= 1 && N >= kGT && N % kGT == 0 && K >= kGK && K % kGK == 0;
}

bool layernorm_width_ok(int N) {
  const int c = N / 256;
  return N % 256 == 0 && (c == 1 || c == 2 || c == 3 || c == 4 || c == 8 || c == 16);
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
  if (!gemm_shape_ok(g.M, g.N, g.K)) return hipErrorInvalidValue;
  switch (g.dtype) {
    case 1: return gemm_t<f16>(g, st);
    case 2: return gemm_t<bf16>(g, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_layernorm(int dtype, const float* z, const void* gamma, const void* beta,
                            float eps, int M, int N, float* out_f32, void* out_t,
                            hipStream_t st) {
  if (!layernorm_width_ok(N)) return hipErrorInvalidValue;
  switch (dtype) {
    case 1: return layernorm_t<f16>(z, gamma, beta, eps, M, N, out_f32, out_t, st);
    case 2: return layernorm_t<bf16>(z, gamma, beta, eps, M, N, out_f32, out_t, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace lf

// Preprocessing kernels: global-token index compaction and local-mask shift.
//
// [FT-LF] = the page "FasterTransformer Longformer 推理加速实践：PyTorch 集成、输入约束与
// 端到端性能解析", section "Longformer Encoder 计算流程", preprocessing items 1 and 2.
//
// Compaction design (gfx950): each batch row is cut into chunks of kChunkMin (or
// more, so that a row has at most kMaxChunks) positions, one 256-thread workgroup
// per chunk, so a row's work spreads over many CUs.  A workgroup needs the number of
// flagged positions before its chunk; it counts them itself from the mask (16-byte
// loads of the row's earlier part, all issued before any is used), so no workgroup
// waits for another.  Inside the chunk, passes of 1024 positions (four 256-wide
// slices): every wave takes a 64-bit ballot of its flags, the per-wave popcounts
// (4 slices x 4 waves = 16 values, in position order) are scanned by one wave, and
// each lane's rank is carry + wave offset + popcount of the ballot bits below it.
// Flagged positions go to the front in ascending order, the others to the back in
// descending order.  The shift and the zeroing of the attention tickets are spread
// over the same workgroups.
#include <cstdint>

#include "lf_device.h"
#include "lf_internal.h"

namespace lf {

namespace {

constexpr int kPrepThreads = 256;
constexpr int kPrepWaves = kPrepThreads / 64;
constexpr int kSlices = 4;
constexpr int kPass = kSlices * kPrepThreads;   // positions per pass
constexpr int kChunkMin = kPass;                // positions per workgroup, at least
constexpr int kMaxChunks = 64;                  // workgroups per batch row, at most
constexpr int kCountBatch = 8;                  // 16-byte loads in flight per thread

// A global-mask value flags a global token iff it is +0 or -0 (every bit but the
// sign clear); the count and the partition use this one test.
__device__ inline bool zero_bits(float x) { return (__float_as_uint(x) & 0x7fffffffu) == 0u; }
__device__ inline bool zero_bits(f16 x) { return (__builtin_bit_cast(uint16_t, x) & 0x7fffu) == 0u; }
__device__ inline bool zero_bits(bf16 x) { return (__builtin_bit_cast(uint16_t, x) & 0x7fffu) == 0u; }

// Zeros among the 16 bytes w holding elements of size E.
template <int E>
__device__ inline int zeros16(const u32x4& w) {
  int c = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (E == 2)
      c += ((w[k] & 0x7fffu) == 0u) + ((w[k] & 0x7fff0000u) == 0u);
    else
      c += (w[k] & 0x7fffffffu) == 0u;
  }
  return c;
}

// Sum of one int per thread over the workgroup (every thread gets it).
__device__ inline int block_sum(int x) {
  __shared__ int s_part[kPrepWaves];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  __syncthreads();   // earlier readers of s_part are done
  if (lane_id() == 0) s_part[threadIdx.x >> 6] = x;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < kPrepWaves; ++w) t += s_part[w];
  return t;
}

// Flagged positions among row[0 .. c0): c0 is a multiple of kChunkMin, so of the 16-
// byte vector length; rows that are not 16-byte aligned take 2- or 4-byte loads.
template <typename T>
__device__ inline int count_before(const T* __restrict__ row, int c0) {
  constexpr int kV = 16 / (int)sizeof(T);
  const int tid = threadIdx.x;
  int cnt = 0;
  if ((reinterpret_cast<uintptr_t>(row) & 15u) == 0u) {
    const u32x4* rv = reinterpret_cast<const u32x4*>(row);
    const int nv = c0 / kV;
    for (int base = 0; base < nv; base += kCountBatch * kPrepThreads) {
      u32x4 w[kCountBatch];
#pragma unroll
      for (int k = 0; k < kCountBatch; ++k) {
        const int i = base + k * kPrepThreads + tid;
        w[k] = i < nv ? rv[i] : u32x4{~0u, ~0u, ~0u, ~0u};   // all ones: no zero
      }
#pragma unroll
      for (int k = 0; k < kCountBatch; ++k) cnt += zeros16<(int)sizeof(T)>(w[k]);
    }
  } else {
    for (int base = 0; base < c0; base += kCountBatch * kPrepThreads) {
      bool z[kCountBatch];
#pragma unroll
      for (int k = 0; k < kCountBatch; ++k) {
        const int i = base + k * kPrepThreads + tid;
        z[k] = i < c0 && zero_bits(row[i]);
      }
#pragma unroll
      for (int k = 0; k < kCountBatch; ++k) cnt += z[k];
    }
  }
  return block_sum(cnt);
}

template <typename T, bool PART, bool SHIFT>
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(const T* __restrict__ gmask,
                                                            const T* __restrict__ lmask, int S,
                                                            int n_chunks, int chunk,
                                                            int32_t* __restrict__ gidx,
                                                            int32_t* __restrict__ gcnt,
                                                            T* __restrict__ bias,
                                                            int* __restrict__ tickets,
                                                            int tickets_per_row) {
  const int b = blockIdx.x / n_chunks;
  const int ch = blockIdx.x % n_chunks;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // zero the attention kernel's per-(b, h) tickets of this batch row
  if (tickets)
    for (int i = ch * kPrepThreads + tid; i < tickets_per_row; i += n_chunks * kPrepThreads)
      tickets[(size_t)b * tickets_per_row + i] = 0;
  const int c0 = ch * chunk;
  const int c1 = min(S, c0 + chunk);
  const T* gm = gmask + (size_t)b * S;
  const T* lm = lmask + (size_t)b * S;
  if (SHIFT) {
    T* bo = bias + (size_t)b * S;
    for (int base = c0; base < c1; base += kPass) {
      T lv[kSlices];
#pragma unroll
      for (int e = 0; e < kSlices; ++e) {
        const int pos = base + e * kPrepThreads + tid;
        lv[e] = pos < c1 ? lm[pos] : Elem<T>::from_f(0.0f);
      }
#pragma unroll
      for (int e = 0; e < kSlices; ++e) {
        const int pos = base + e * kPrepThreads + tid;
        if (pos < c1) bo[pos] = Elem<T>::from_f(fmaf(Elem<T>::to_f(lv[e]), 10000.0f, -10000.0f));
      }
    }
  }
  if (!PART) return;
  __shared__ int s_off[kSlices * kPrepWaves];
  __shared__ int s_total;
  int32_t* out = gidx + (size_t)b * S;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // the first pass's flags go out before the count of the earlier positions
  T gv[kSlices];
#pragma unroll
  for (int e = 0; e < kSlices; ++e) {
    const int pos = c0 + e * kPrepThreads + tid;
    gv[e] = pos < c1 ? gm[pos] : Elem<T>::from_f(1.0f);
  }
  int carry = count_before<T>(gm, c0);
  for (int base = c0; base < c1; base += kPass) {
    if (base != c0) {
#pragma unroll
      for (int e = 0; e < kSlices; ++e) {
        const int pos = base + e * kPrepThreads + tid;
        gv[e] = pos < c1 ? gm[pos] : Elem<T>::from_f(1.0f);
      }
    }
    bool f[kSlices];
    uint64_t bal[kSlices];
#pragma unroll
    for (int e = 0; e < kSlices; ++e) {
      const int pos = base + e * kPrepThreads + tid;
      f[e] = pos < c1 && zero_bits(gv[e]);
      bal[e] = __ballot(f[e]);
    }
    if (lane == 0) {
#pragma unroll
      for (int e = 0; e < kSlices; ++e) s_off[e * kPrepWaves + wave] = __popcll(bal[e]);
    }
    __syncthreads();
    if (wave == 0) {
      const int x = lane < kSlices * kPrepWaves ? s_off[lane] : 0;
      const int ex = wave_excl_scan(x);
      if (lane < kSlices * kPrepWaves) s_off[lane] = ex;
      if (lane == kSlices * kPrepWaves - 1) s_total = ex + x;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kSlices; ++e) {
      const int pos = base + e * kPrepThreads + tid;
      if (pos < c1) {
        const int before = carry + s_off[e * kPrepWaves + wave] + __popcll(bal[e] & below);
        if (f[e])
          out[before] = pos;
        else
          out[S - 1 - (pos - before)] = pos;
      }
    }
    carry += s_total;
    __syncthreads();
  }
  if (ch == n_chunks - 1 && tid == 0) gcnt[b] = carry;
}

// Elementwise shift over n values, 8 per thread per step (16-byte loads for 16-bit types).
template <typename T>
__global__ __launch_bounds__(256) void mask_shift_kernel(const T* __restrict__ m, int64_t n,
                                                         T* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 8;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8; i < n; i += stride) {
    if (i + 8 <= n) {
      T x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = m[i + e];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        out[i + e] = Elem<T>::from_f(fmaf(Elem<T>::to_f(x[e]), 10000.0f, -10000.0f));
    } else {
      for (int64_t j = i; j < n; ++j)
        out[j] = Elem<T>::from_f(fmaf(Elem<T>::to_f(m[j]), 10000.0f, -10000.0f));
    }
  }
}

// Precondition checker: one workgroup per batch row.  flags[0..3] get
// 1 + smallest offending flat index (atomicMin over a 0-means-none encoding is
// done as atomicMin on (index+1) after the host preset them to INT_MAX).
template <typename T>
__global__ __launch_bounds__(256) void check_masks_kernel(const T* __restrict__ lm,
                                                          const T* __restrict__ gm, int S, int G,
                                                          int* __restrict__ flags) {
  const int b = blockIdx.x;
  __shared__ int s_first_non_global;
  __shared__ int s_count;
  if (threadIdx.x == 0) {
    s_first_non_global = S;
    s_count = 0;
  }
  __syncthreads();
  const T notg = Elem<T>::from_f(-10000.0f);
  for (int s = threadIdx.x; s < S; s += blockDim.x) {
    const size_t i = (size_t)b * S + s;
    const float l = Elem<T>::to_f(lm[i]);
    const T graw = gm[i];
    const float g = Elem<T>::to_f(graw);
    if (!(l == 0.0f || l == 1.0f)) atomicMin(&flags[0], (int)(i + 1));
    const bool is_g = (g == 0.0f);
    if (!is_g && !(g == Elem<T>::to_f(notg))) atomicMin(&flags[1], (int)(i + 1));
    if (is_g)
      atomicAdd(&s_count, 1);
    else
      atomicMin(&s_first_non_global, s);
  }
  __syncthreads();
  // globals are leading iff every flagged position precedes the first unflagged one,
  // i.e. count == first unflagged position (or S when none)
  if (threadIdx.x == 0) {
    const int n = s_count;
    const int first = s_first_non_global;
    if (n != (first < S ? first : S)) atomicMin(&flags[2], b + 1);
    if (n > G) atomicMin(&flags[3], b + 1);
  }
}

// n ints set to v (a kernel rather than hipMemsetAsync, so that a caller may capture
// it in a graph).
__global__ __launch_bounds__(256) void fill_i32_kernel(int* __restrict__ p, int64_t n, int v) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

// Positions per workgroup of the compaction: kChunkMin, or a multiple of it that
// keeps a row at kMaxChunks workgroups.
inline int prep_chunk(int S) {
  const int passes = (S + kChunkMin - 1) / kChunkMin;
  const int per = (passes + kMaxChunks - 1) / kMaxChunks;
  return (per < 1 ? 1 : per) * kChunkMin;
}

template <typename T>
hipError_t prep_t(const void* g, const void* l, int B, int S, int32_t* idx, int32_t* cnt,
                  void* bias, int* tickets, int tickets_per_row, hipStream_t st) {
  const int chunk = prep_chunk(S);
  const int n_chunks = (S + chunk - 1) / chunk;
  const int64_t grid = (int64_t)B * n_chunks;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (g && l)
    prep_kernel<T, true, true><<<(unsigned)grid, kPrepThreads, 0, st>>>(
        (const T*)g, (const T*)l, S, n_chunks, chunk, idx, cnt, (T*)bias, tickets, tickets_per_row);
  else if (g)
    prep_kernel<T, true, false><<<(unsigned)grid, kPrepThreads, 0, st>>>(
        (const T*)g, nullptr, S, n_chunks, chunk, idx, cnt, nullptr, tickets, tickets_per_row);
  else
    prep_kernel<T, false, true><<<(unsigned)grid, kPrepThreads, 0, st>>>(
        nullptr, (const T*)l, S, n_chunks, chunk, nullptr, nullptr, (T*)bias, tickets,
        tickets_per_row);
  return hipGetLastError();
}

template <typename T>
hipError_t shift_t(const void* m, int64_t n, void* out, hipStream_t st) {
  int64_t blocks = (n + 256 * 8 - 1) / (256 * 8);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  mask_shift_kernel<T><<<(int)blocks, 256, 0, st>>>((const T*)m, n, (T*)out);
  return hipGetLastError();
}

template <typename T>
hipError_t check_t(const void* l, const void* g, int B, int S, int G, int* flags,
                   hipStream_t st) {
  check_masks_kernel<T><<<B, 256, 0, st>>>((const T*)l, (const T*)g, S, G, flags);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prep(int dtype, const void* global_mask, const void* local_mask, int B, int S,
                       int32_t* gidx, int32_t* gcnt, void* bias, int* tickets,
                       int tickets_per_row, hipStream_t st) {
  switch (dtype) {
    case 0: return prep_t<float>(global_mask, local_mask, B, S, gidx, gcnt, bias, tickets, tickets_per_row, st);
    case 1: return prep_t<f16>(global_mask, local_mask, B, S, gidx, gcnt, bias, tickets, tickets_per_row, st);
    case 2: return prep_t<bf16>(global_mask, local_mask, B, S, gidx, gcnt, bias, tickets, tickets_per_row, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fill_i32(int* p, int64_t n, int v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  fill_i32_kernel<<<(int)blocks, 256, 0, st>>>(p, n, v);
  return hipGetLastError();
}

hipError_t launch_mask_shift(int dtype, const void* local_mask, int64_t n, void* bias,
                             hipStream_t st) {
  switch (dtype) {
    case 0: return shift_t<float>(local_mask, n, bias, st);
    case 1: return shift_t<f16>(local_mask, n, bias, st);
    case 2: return shift_t<bf16>(local_mask, n, bias, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_check_masks(int dtype, const void* local_mask, const void* global_mask, int B,
                              int S, int G, int* flags, hipStream_t st) {
  switch (dtype) {
    case 0: return check_t<float>(local_mask, global_mask, B, S, G, flags, st);
    case 1: return check_t<f16>(local_mask, global_mask, B, S, G, flags, st);
    case 2: return check_t<bf16>(local_mask, global_mask, B, S, G, flags, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace lf

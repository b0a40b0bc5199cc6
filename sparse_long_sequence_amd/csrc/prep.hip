// Preprocessing kernels: global-token index compaction and local-mask shift.
//
// [FT-LF] = the page "FasterTransformer Longformer 推理加速实践：PyTorch 集成、输入约束与
// 端到端性能解析", section "Longformer Encoder 计算流程", preprocessing items 1 and 2.
//
// Compaction design (gfx950): one 1024-thread workgroup per batch row.  Each pass
// covers 4096 positions as four 1024-wide slices; inside a slice every wave takes a
// 64-bit ballot of its flags, the per-wave popcounts (4 slices x 16 waves = 64
// values, in position order) are scanned by one wave, and each lane's rank is
// carry + wave offset + popcount of the ballot bits below it.  Flagged positions go
// to the front in ascending order, the others to the back in descending order.
#include "lf_device.h"
#include "lf_internal.h"

namespace lf {

namespace {

constexpr int kPrepThreads = 1024;
constexpr int kPrepWaves = kPrepThreads / 64;
constexpr int kSlices = 4;

template <typename T, bool PART, bool SHIFT>
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(const T* __restrict__ gmask,
                                                            const T* __restrict__ lmask, int S,
                                                            int32_t* __restrict__ gidx,
                                                            int32_t* __restrict__ gcnt,
                                                            T* __restrict__ bias,
                                                            int* __restrict__ tickets,
                                                            int tickets_per_row) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // zero the attention kernel's per-(b, h) tickets of this batch row
  if (tickets)
    for (int i = tid; i < tickets_per_row; i += kPrepThreads)
      tickets[(size_t)b * tickets_per_row + i] = 0;
  __shared__ int s_off[kSlices * kPrepWaves];
  __shared__ int s_total;
  const T* gm = gmask + (size_t)b * S;
  const T* lm = lmask + (size_t)b * S;
  int32_t* out = gidx + (size_t)b * S;
  T* bo = bias + (size_t)b * S;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int carry = 0;
  for (int base = 0; base < S; base += kSlices * kPrepThreads) {
    // every load of the pass is issued before any result is used
    T gv[kSlices], lv[kSlices];
#pragma unroll
    for (int e = 0; e < kSlices; ++e) {
      const int pos = base + e * kPrepThreads + tid;
      if (PART) gv[e] = pos < S ? gm[pos] : Elem<T>::from_f(1.0f);
      if (SHIFT) lv[e] = pos < S ? lm[pos] : Elem<T>::from_f(0.0f);
    }
    if (SHIFT) {
#pragma unroll
      for (int e = 0; e < kSlices; ++e) {
        const int pos = base + e * kPrepThreads + tid;
        if (pos < S) bo[pos] = Elem<T>::from_f(fmaf(Elem<T>::to_f(lv[e]), 10000.0f, -10000.0f));
      }
    }
    if (PART) {
      bool f[kSlices];
      uint64_t bal[kSlices];
#pragma unroll
      for (int e = 0; e < kSlices; ++e) {
        f[e] = Elem<T>::to_f(gv[e]) == 0.0f;
        bal[e] = __ballot(f[e]);
      }
      if (lane == 0) {
#pragma unroll
        for (int e = 0; e < kSlices; ++e) s_off[e * kPrepWaves + wave] = __popcll(bal[e]);
      }
      __syncthreads();
      if (wave == 0) {
        const int x = s_off[lane];
        const int ex = wave_excl_scan(x);
        s_off[lane] = ex;
        if (lane == 63) s_total = ex + x;
      }
      __syncthreads();
#pragma unroll
      for (int e = 0; e < kSlices; ++e) {
        const int pos = base + e * kPrepThreads + tid;
        if (pos < S) {
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
  }
  if (PART && tid == 0) gcnt[b] = carry;
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

template <typename T>
hipError_t prep_t(const void* g, const void* l, int B, int S, int32_t* idx, int32_t* cnt,
                  void* bias, int* tickets, int tickets_per_row, hipStream_t st) {
  if (g && l)
    prep_kernel<T, true, true><<<B, kPrepThreads, 0, st>>>((const T*)g, (const T*)l, S, idx, cnt,
                                                          (T*)bias, tickets, tickets_per_row);
  else if (g)
    prep_kernel<T, true, false><<<B, kPrepThreads, 0, st>>>((const T*)g, nullptr, S, idx, cnt,
                                                           nullptr, tickets, tickets_per_row);
  else
    prep_kernel<T, false, true><<<B, kPrepThreads, 0, st>>>(nullptr, (const T*)l, S, nullptr,
                                                           nullptr, (T*)bias, tickets,
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

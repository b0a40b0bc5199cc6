// fp32 band + global attention on the vector ALUs (no fp32 matrix path needed at
// the fp32 parity tolerance).
//
// [FT-LF] = the page "FasterTransformer Longformer 推理加速实践", section
// "Longformer Encoder 计算流程", per-layer steps 3-4: local rows normalise over
// their window plus the global tokens, global rows over the whole sequence,
// padded rows are zeroed; the shifted mask is an additive score bias
// (preprocessing item 2).
//
// One 64-lane workgroup owns 64 query slots of one (batch, head): either local
// rows s0..s0+63 or global rows r0..r0+63.  Keys stream through LDS in chunks of
// 64 rows (K and V in fp32); every lane runs an exact online softmax for its own
// query.  Global keys (positions global_idx[0..n_b)) come first for local rows;
// band keys are [max(n_b, s0 - W/2), min(S-1, s0+63+W/2)] when the global tokens
// lead, or [max(0, s0 - W/2), ...] minus the positions whose global-mask value is
// zero when they may sit anywhere (any_pos).
#include "lf_device.h"
#include "lf_internal.h"

namespace lf {

namespace {

constexpr int kRows = 64;
constexpr int kChunk = 64;
constexpr int kLd = 65;  // padded LDS row (floats)

template <typename T>
__device__ inline void stage_rows(const T* __restrict__ src_head, const int32_t* __restrict__ rows,
                                  int first, int count, int S, float* __restrict__ kl,
                                  const T* __restrict__ bias_row, float* __restrict__ bl,
                                  bool gather, const T* __restrict__ excl_row = nullptr) {
  // lane i stages key slot i: row = gather ? rows[first+i] : first+i
  const int i = threadIdx.x;
  int row = -1;
  if (i < count) row = gather ? rows[first + i] : first + i;
  if (row >= S) row = -1;
  const T* src = src_head + (size_t)(row < 0 ? 0 : row) * 64;
  for (int d = 0; d < 64; ++d) kl[i * kLd + d] = row >= 0 ? Elem<T>::to_f(src[d]) : 0.0f;
  // excl_row: a position whose global-mask value is zero is not a band key
  const bool excl = row >= 0 && excl_row && Elem<T>::to_f(excl_row[row]) == 0.0f;
  if (bl) bl[i] = row >= 0 && !excl ? Elem<T>::to_f(bias_row[row]) : -INFINITY;
}

template <typename T>
__global__ __launch_bounds__(64) void attn_valu_kernel(AttnArgs a, int n_local_tiles,
                                                       int n_global_tiles) {
  __shared__ float ks[kChunk * kLd];
  __shared__ float vs[kChunk * kLd];
  __shared__ float bs[kChunk];
  const int lane = threadIdx.x;
  const int tiles_per_head = n_local_tiles + n_global_tiles;
  const int bh = blockIdx.x / tiles_per_head;
  const int tile = blockIdx.x % tiles_per_head;
  const int b = bh / a.H;
  const int h = bh % a.H;
  const int S = a.S;
  const int half = a.W / 2;
  const int nb = a.gcnt[b];
  const size_t head = ((size_t)b * a.H + h) * (size_t)S * 64;
  const T* bias = (const T*)a.bias + (size_t)b * S;
  const int32_t* gidx = a.gidx + (size_t)b * S;
  const bool is_global_tile = tile >= n_local_tiles;
  const T* gmask = a.any_pos ? (const T*)a.global_mask + (size_t)b * S : nullptr;

  int s;            // output position of this lane's row
  bool active;      // lane owns a row this kernel computes
  const T* qrow;
  if (!is_global_tile) {
    const int s0 = tile * kRows;
    s = s0 + lane;
    active = s < S && (gmask ? Elem<T>::to_f(gmask[s]) != 0.0f : s >= nb);
    qrow = (const T*)a.q + head + (size_t)(active ? s : 0) * 64;
  } else {
    const int r = (tile - n_local_tiles) * kRows + lane;
    active = r < nb;
    s = active ? gidx[r] : 0;
    qrow = (const T*)a.qg + (((size_t)b * a.H + h) * a.G + (active ? r : 0)) * 64;
  }
  if (__ballot(active) == 0ull) return;

  float qv[64];
  for (int d = 0; d < 64; ++d) qv[d] = active ? Elem<T>::to_f(qrow[d]) * a.scale : 0.0f;
  float acc[64];
  for (int d = 0; d < 64; ++d) acc[d] = 0.0f;
  float m = -INFINITY, l = 0.0f;

  auto consume = [&](int nkeys, int key0, bool band) {
    for (int i = 0; i < nkeys; ++i) {
      float sc = 0.0f;
      for (int d = 0; d < 64; ++d) sc = fmaf(qv[d], ks[i * kLd + d], sc);
      sc += bs[i];
      bool ok = active && bs[i] != -INFINITY;
      if (band) {
        const int j = key0 + i;
        ok = ok && (j - s <= half) && (s - j <= half);
      }
      if (ok) {
        const float mn = fmaxf(m, sc);
        const float alpha = expf(m - mn);
        const float p = expf(sc - mn);
        l = l * alpha + p;
        for (int d = 0; d < 64; ++d) acc[d] = fmaf(p, vs[i * kLd + d], acc[d] * alpha);
        m = mn;
      }
    }
  };

  if (!is_global_tile) {
    const T* kh = (const T*)a.k + head;
    const T* vh = (const T*)a.v + head;
    // global keys, gathered by index
    for (int c0 = 0; c0 < nb; c0 += kChunk) {
      const int cnt = min(kChunk, nb - c0);
      __syncthreads();
      stage_rows<T>(kh, gidx, c0, cnt, S, ks, bias, bs, true);
      stage_rows<T>(vh, gidx, c0, cnt, S, vs, bias, nullptr, true);
      __syncthreads();
      consume(cnt, 0, false);
    }
    const int s0 = tile * kRows;
    const int lo = max(gmask ? 0 : nb, s0 - half);
    const int hi = min(S - 1, s0 + kRows - 1 + half);
    for (int kb = lo; kb <= hi; kb += kChunk) {
      const int cnt = min(kChunk, hi - kb + 1);
      __syncthreads();
      stage_rows<T>(kh, nullptr, kb, cnt, S, ks, bias, bs, false, gmask);
      stage_rows<T>(vh, nullptr, kb, cnt, S, vs, bias, nullptr, false);
      __syncthreads();
      consume(cnt, kb, true);
    }
  } else {
    const T* kh = (const T*)a.kg + head;
    const T* vh = (const T*)a.vg + head;
    for (int kb = 0; kb < S; kb += kChunk) {
      const int cnt = min(kChunk, S - kb);
      __syncthreads();
      stage_rows<T>(kh, nullptr, kb, cnt, S, ks, bias, bs, false);
      stage_rows<T>(vh, nullptr, kb, cnt, S, vs, bias, nullptr, false);
      __syncthreads();
      consume(cnt, kb, false);
    }
  }
  if (!active) return;
  const bool live = Elem<T>::to_f(bias[s]) == 0.0f;
  T* o = (T*)a.out + (size_t)b * a.out_sb + (size_t)h * a.out_sh + (size_t)s * a.out_ss;
  const float inv = live ? 1.0f / l : 0.0f;
  for (int d = 0; d < 64; ++d) o[d] = Elem<T>::from_f(live ? acc[d] * inv : 0.0f);
}

}  // namespace

hipError_t launch_attention_fp32(const AttnArgs& a, hipStream_t st) {
  const int n_local = (a.S + kRows - 1) / kRows;
  const int n_global = (a.G + kRows - 1) / kRows;
  const int64_t grid = (int64_t)a.B * a.H * (n_local + n_global);
  if (a.ev_begin) {
    hipError_t e0 = hipEventRecord(a.ev_begin, st);
    if (e0 != hipSuccess) return e0;
  }
  switch (a.dtype) {
    case 0: attn_valu_kernel<float><<<(unsigned)grid, 64, 0, st>>>(a, n_local, n_global); break;
    case 1: attn_valu_kernel<f16><<<(unsigned)grid, 64, 0, st>>>(a, n_local, n_global); break;
    case 2: attn_valu_kernel<bf16><<<(unsigned)grid, 64, 0, st>>>(a, n_local, n_global); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && a.ev_end) e = hipEventRecord(a.ev_end, st);
  return e;
}

}  // namespace lf

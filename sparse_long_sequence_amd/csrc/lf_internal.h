// Internal launch interface between the C ABI layer (lf_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lf {

// Everything one attention launch needs.  Output element (b, h, s, d) lives at
// out + b*out_sb + h*out_sh + s*out_ss + d, so the encoder layer can write the
// head-joined [B, S, H*64] layout directly.
struct AttnArgs {
  int dtype;
  int raw;                // 1: read local_mask / global_mask; 0: read gidx / gcnt / bias
  const void *q, *k, *v, *qg, *kg, *vg;
  const void* local_mask;   // [B, S] dtype (raw mode)
  const void* global_mask;  // [B, S] dtype (raw mode)
  const int32_t* gidx;    // [B, S] (pre mode)
  const int32_t* gcnt;    // [B]    (pre mode)
  const void* bias;       // [B, S] shifted local mask, dtype (pre mode)
  void* out;
  int64_t out_sb, out_sh, out_ss;
  int B, H, S, W, G;
  float scale;
  float* partials;        // global-row partial states [B*H][n_split][G][kPartPitch]
  int* counters;          // [B*H] split tickets: zero on entry, left zero on exit
  int n_split;            // key splits of the global rows
  int split_len;          // keys per split (multiple of 128)
  hipEvent_t ev_begin;    // if non-null: recorded right before / after the main kernel
  hipEvent_t ev_end;
};

// Floats per global-row partial state: m (scaled log2 units), l, 2 pad, o[64].
constexpr int kPartPitch = 68;

// Key splits of the global rows for sequence length S (fp16 / bf16 kernel).
void attn_split_plan(int S, int* n_split, int* split_len);

// Global-index partition + count (when global_mask != NULL), mask shift (when
// local_mask != NULL) and, when tickets != NULL, zeroing of B * tickets_per_row
// attention tickets; one launch.
hipError_t launch_prep(int dtype, const void* global_mask, const void* local_mask, int B, int S,
                       int32_t* gidx, int32_t* gcnt, void* bias, int* tickets,
                       int tickets_per_row, hipStream_t st);
hipError_t launch_mask_shift(int dtype, const void* local_mask, int64_t n, void* bias,
                             hipStream_t st);
hipError_t launch_attention(const AttnArgs& a, hipStream_t st);
hipError_t launch_attention_fp32(const AttnArgs& a, hipStream_t st);

// Mask precondition check: writes 4 ints to `flags` (device): bad local value,
// bad global value, non-leading global, count > G; each holds 1 + first offending
// flat index (0 = no violation).
hipError_t launch_check_masks(int dtype, const void* local_mask, const void* global_mask, int B,
                              int S, int G, int* flags, hipStream_t st);

// Layer pieces.
hipError_t launch_gemm(int dtype, int epilogue, const void* A, int lda, const void* Bw, int ldb,
                       const void* bias, const void* resid_f32, void* C, int ldc, int M, int N,
                       int K, int a_rows_per_batch, int a_batch_stride_rows, void* aux0,
                       void* aux1, void* aux2, void* aux3, void* aux4, int S, int H,
                       hipStream_t st);
hipError_t launch_layernorm(int dtype, const float* z, const void* gamma, const void* beta,
                            float eps, int M, int N, float* out_f32, void* out_t,
                            hipStream_t st);

}  // namespace lf

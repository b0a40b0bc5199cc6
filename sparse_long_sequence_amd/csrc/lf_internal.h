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
  int any_pos;            // 1: global tokens at any positions (raw mode on fp16 / bf16, pre
                          // mode on fp32): band keys and output rows test global_mask, global
                          // keys and rows go through gidx / gcnt
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
  int wg_per_gen;         // workgroups the dispatcher places before any CU gets a second
                          // (the CU count; set by the launch): in the 4-wave layout,
                          // consecutive generations pair up on the CUs
  hipEvent_t ev_begin;    // if non-null: recorded right before / after the main kernel
  hipEvent_t ev_end;
};

// lf_attn_forward's computation in memory the caller provides (lf_api.hip): `scratch`
// (device, 256-byte aligned, scratch_bytes >= attn_forward_scratch_bytes) holds the
// global-row partials (fp16 / bf16) or the preprocessed masks (fp32); `tickets` (device,
// ticket_capacity ints, zero on entry and left zero) the split tickets.  Validates the
// arguments as lf_attn_forward does; returns an lf_status, with the message for
// lf_last_error() naming `who`.
size_t attn_forward_scratch_bytes(int dtype, int B, int H, int S, int G);
// The argument checks of attn_forward_in alone (nothing is enqueued).
int attn_forward_validate(int dtype, const void* q, const void* k, const void* v,
                          const void* qg, const void* kg, const void* vg, const void* local_mask,
                          const void* global_mask, int B, int H, int S, int W, int G,
                          const void* out, size_t scratch_bytes, int ticket_capacity,
                          const char* who);
int attn_forward_in(int dtype, const void* q, const void* k, const void* v, const void* qg,
                    const void* kg, const void* vg, const void* local_mask,
                    const void* global_mask, int B, int H, int S, int W, int G, void* out,
                    void* stream, char* scratch, size_t scratch_bytes, int* tickets,
                    int ticket_capacity, const char* who);
// Records a failure for lf_last_error(); returns code.
int set_error(int code, const char* msg);

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
// n ints at p set to v, one launch (no memset node).
hipError_t launch_fill_i32(int* p, int64_t n, int v, hipStream_t st);
hipError_t launch_attention(const AttnArgs& a, hipStream_t st);
// The attention kernel with one extra workgroup per (b, h) for the global rows (grid =
// band tiles + B * H; a.n_split == 1): attn_mfma_gwg.hip.
hipError_t launch_attention_gwg(const AttnArgs& a, int n_tiles, unsigned grid, hipStream_t st);
// The 4-wave layout (attn_mfma_w4.hip): 128-row workgroups, two per CU; split plan as
// attn_split_plan gives it for long sequences.
hipError_t launch_attention_w4(const AttnArgs& a, hipStream_t st);
hipError_t launch_attention_fp32(const AttnArgs& a, hipStream_t st);

// Mask precondition check: writes 4 ints to `flags` (device): bad local value,
// bad global value, non-leading global, count > G; each holds 1 + first offending
// flat index (0 = no violation).
hipError_t launch_check_masks(int dtype, const void* local_mask, const void* global_mask, int B,
                              int S, int G, int* flags, hipStream_t st);

// Layer pieces (gemm.hip).  C[m, n] = sum_k A[arow(m), k] * W[n, k] + bias[n], with
// arow(m) = (m / a_group) * a_group_stride + m % a_group when a_group > 0 (or that
// group's a_rows entry, see GemmArgs), else m;
// then the epilogue.  A, W, bias, outputs and the T residual are in the layer dtype.
enum GemmEpi {
  kEpiHeads = 0,     // n -> tensor n / D, head (n % D) / 64, dim n % 64; m -> (m / rows,
                     // m % rows): heads[tensor][((b * H + h) * rows + r) * 64 + d]
  kEpiGelu = 1,      // out[m * ldo + n] = gelu(acc + bias), dtype
  kEpiResidT = 2,    // out[m * ldo + n] = acc + bias + resid[m * ldr + n] (resid dtype), fp32
  kEpiResidF32 = 3,  // same with an fp32 residual
  kEpiPartial = 4,   // split-K: part[split][m * N + n] = acc (fp32, no bias); reduced by
                     // launch_layernorm_parts
};

struct GemmArgs {
  int dtype, epi;
  const void* a;
  int lda, a_group, a_group_stride;
  const void* w;
  int ldw;
  const void* bias;
  int M, N, K;
  void* heads[5];
  int D, H, rows;
  void* out;
  int ldo;
  const void* resid;
  int ldr;
  int splits;            // split-K factor (kEpiPartial; else 1): split s sums k in
                         // [s K / splits, (s + 1) K / splits)
  float* part;           // kEpiPartial output: [splits][M][N] fp32
  const int32_t* a_rows; // optional with a_group > 0: arow(m) = (m / a_group) *
                         // a_group_stride + a_rows[(m / a_group) * a_group_stride + m %
                         // a_group] (the global-query rows gathered through the index)
};

// N a positive multiple of 128, K of 64, M >= 1.
bool gemm_shape_ok(int M, int N, int K);
// Split-K factor for a GEMM whose 128 x 128 grid would leave CUs idle: the smallest
// power of two (up to 16) that brings the grid to 256 workgroups, with K / splits a
// multiple of 64; 1 when the grid is large enough.
int gemm_splits(int M, int N, int K);
// Row widths the LayerNorm kernel takes (multiples of 256 up to 4096).
bool layernorm_width_ok(int N);
hipError_t launch_gemm(const GemmArgs& g, hipStream_t st);
// Two head-split GEMMs (kEpiHeads, no split-K, same dtype and K) in one launch: the
// tiles of g2 follow those of g in the grid (g's tile shape), so a small g2 fills
// the idle slots of g's last round of tiles.
hipError_t launch_gemm_pair(const GemmArgs& g, const GemmArgs& g2, hipStream_t st);
// LayerNorm of z = sum_s part[s] + bias + resid (resid in the layer dtype, or fp32
// when resid_f32): the reduction of a split-K GEMM fused into the row kernel.
hipError_t launch_layernorm_parts(int dtype, const float* part, int splits, const void* bias,
                                  const void* resid, bool resid_f32, const void* gamma,
                                  const void* beta, float eps, int M, int N, float* out_f32,
                                  void* out_t, hipStream_t st);
// Fused FFN (gemm.hip): part[s][m][:] = GELU(x[m] W1^T + b1) W2^T over F slice s of
// `splits` equal slices, the GELU output kept on chip; fp16 / bf16, D in
// {256, 512, 768, 1024}, F a multiple of 32 * splits.
int ffn_fused_splits(int M, int F);
bool ffn_fused_ok(int dtype, int D, int F, int splits);
hipError_t launch_ffn_fused(int dtype, const void* x, const void* w1, const void* b1,
                            const void* w2, int M, int D, int F, int splits, float* part,
                            hipStream_t st);
hipError_t launch_layernorm(int dtype, const float* z, const void* gamma, const void* beta,
                            float eps, int M, int N, float* out_f32, void* out_t,
                            hipStream_t st);

}  // namespace lf

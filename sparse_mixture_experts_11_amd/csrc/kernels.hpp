// Internal launch interface between the C ABI (moe_api.hip) and the kernels.
// Every launcher enqueues on `st` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---- router (route.hip) ----------------------------------------------------
// Partial rows [rows][N] of the balance statistics that the router writes
// for this layer (one per wave, per block or per token, by kernel).
int route_waves(int64_t T, int N, int d, bool u_bf16, bool w_bf16);
// Wave-per-token-group router for N <= 64: scores, softmax, top-k, weights.
// bias: optional [N] selection bias (top-k of z + bias; weights from the
// unbiased softmax).
hipError_t launch_route_wave(const void *u, bool u_bf16, const void *W, bool w_bf16, int64_t T,
                             int d, int N, int k, int gate, const float *bias, int32_t *idx,
                             float *w, float *part_p, int32_t *part_cnt, hipStream_t st);
// Softmax + top-k from materialised fp32 logits [T, N] (N <= 1024).
hipError_t launch_topk_logits(const float *logits, const float *logits2, int64_t T, int N, int k,
                              int gate, const float *bias, int32_t *idx, float *w, float *part_p,
                              int32_t *part_cnt, hipStream_t st);
// f, P, N sum fP, alpha N sum fP from the per-wave partials (which it
// overwrites: each 32-row slice's sums are left in the slice's first row).
hipError_t launch_stats_finalize(float *part_p, int32_t *part_cnt, int waves, int64_t T, int N,
                                 float alpha, float *stats, hipStream_t st);

// ---- dispatch (dispatch.hip) ----------------------------------------------
int dispatch_blocks(int64_t entries);
// With stats != nullptr the count launch also sums the router's partial
// rows [rows][N] in slices of 64 (extra blocks; each slice's sums overwrite
// its first row) and the scan launch adds the slices and finishes f, P,
// N sum f P and alpha N sum f P: the statistics cost no launch of their own.
hipError_t launch_dispatch(const int32_t *idx, int64_t T, int k, int N, int capacity,
                           int32_t *counts, int32_t *offsets, int32_t *kept_offsets,
                           int32_t *perm, int32_t *row_of, uint8_t *drop,
                           int32_t *blk_counts, float *part_p, int32_t *part_cnt,
                           int rows, float alpha, float *stats, hipStream_t st);
// At most 1024 entries and 1024 experts: one launch does the balance
// statistics (when stats != nullptr, from the router's partial rows) and
// the whole dispatch (when perm != nullptr).
bool small_tail_fits(int64_t entries, int N);
hipError_t launch_small_tail(const float *part_p, const int32_t *part_cnt, int waves, int64_t T,
                             float alpha, float *stats, const int32_t *idx, int k, int N,
                             int capacity, int32_t *counts, int32_t *offsets,
                             int32_t *kept_offsets, int32_t *perm, int32_t *row_of,
                             uint8_t *drop, hipStream_t st);

// ---- grouped GEMM on bf16 MFMA (gemm.hip) -----------------------------------
enum GemmMode { GM_GATHER = 0, GM_SEGMENT = 1, GM_DENSE = 2 };
// EP_GU (backward): the GLU tile's gate and up sums stored as bf16 (out,
// out2).  EP_GLU_BWD (backward): the product is dH; with G = gsrc, U = usrc
// ([rows][ncols] bf16, row stride ldo / 2) it stores dG to out and dU to out2.
enum GemmEpi {
  EP_GLU = 0, EP_F32 = 1, EP_BF16 = 2, EP_ADD_BF16 = 3, EP_GU = 4, EP_GLU_BWD = 5,
  EP_GLU_SAVE = 6  // EP_GLU that also stores the gate and up sums (bf16) for the backward
};

struct GemmArgs {
  // A: rows of K bf16 values, row stride lda (elements).
  const uint16_t *A;
  int64_t lda;
  // B: per group, rows of K values (K-contiguous); B2 holds the "up" rows
  // of a GLU pair (same layout as B).  Group g starts at g * strideB
  // (elements).  bf16 values, or E4M3 codes when bscale is set: then row n
  // of group g is scaled by bscale[g * ncols + n] (bscale2 for B2).
  const void *B;
  const void *B2;
  int64_t strideB;
  const float *bscale, *bscale2;
  int K;
  int ncols;        // output columns per group (h for GLU)
  int mode;         // GemmMode
  int G;            // groups
  int64_t M_dense;  // rows per group in GM_DENSE
  int64_t a_group_rows;  // GM_DENSE: A row offset between groups (0: shared A)
  int kslots;       // k, to turn perm entries into token rows (GM_GATHER)
  const int32_t *perm, *offsets, *kept_offsets;
  const int32_t *tile_start;  // [G+1] m-tile prefix (GM_GATHER / GM_SEGMENT)
  void *out;
  int64_t ldo;
  int64_t out_group_stride;   // GM_DENSE: rows of output per group
  const float *add0, *add1;   // EP_ADD_BF16: out = acc + add0 + add1 (fp32, ldo)
  int act;                    // 0 SwiGLU, 1 SiTU-GLU
  float beta_g, beta_u;
  int bm;                     // m-tile height: 192, else 256
  void *out2;                 // EP_GU: up sums; EP_GLU_BWD: dU; EP_GLU_SAVE: [G | U]
                              // rows of stride ldg (U at column offset ncols)
  const uint16_t *gsrc, *usrc;  // EP_GLU_BWD: G and U
  int64_t ldg;                // EP_GLU_BWD, EP_GLU_SAVE: row stride of G and U (elements)
  // K segments (dense tiles, every group's own k range): group g reduces over
  // k in [kseg[g], kseg[g+1]) (multiples of 64, at least 128), B rows have
  // stride ldb.  Used with EP_F32 for the experts' weight gradients.
  const int32_t *kseg;
  int64_t ldb;
  // Transposed B (bt != 0): B_g stored [K][ldbt], element (n, k) at
  // k * ldbt + n (the weights as the forward keeps them, read without a
  // transposed copy).  With ksplit > 0, k >= ksplit comes from B2 at row
  // k - ksplit (the stacked [W_gate ; W_up] of the dx product).
  int bt;
  int64_t ldbt;
  int ksplit;
  // MXFP4 weights (mx4 != 0, EP_GLU / EP_F32): B holds packed E2M1 pairs
  // (row n of group g at byte (g * strideB + n * K) / 2) and bscale /
  // bscale2 point at E8M0 bytes [G][ncols][K/32].
  int mx4;
  // Dense split-K (kchunk > 0, EP_F32, GM_DENSE, kseg null): group g
  // reduces k in [g kchunk, (g + 1) kchunk) (a multiple of 128) of the same
  // A rows and B rows (row stride ldb) into its own output block of
  // out_group_stride rows; the caller adds the G partial products.
  int kchunk;
};
// m-tile height for groups of about rows_per_group rows (192 or 256).
int gemm_pick_bm(double rows_per_group);
// Upper bound of m-tiles (host side, no device sync).
int64_t gemm_mtile_bound(int64_t rows_total, int groups, int bm);
hipError_t launch_tile_prefix(const int32_t *kept_offsets, int G, int bm, int32_t *tile_start,
                              hipStream_t st);
hipError_t launch_gemm(const GemmArgs &a, int epi, int64_t mtiles_bound, hipStream_t st);

// ---- Quantile Balancing (qb.hip) -------------------------------------------
// One update from the fp32 logits [T, N]: req [N, T] scratch; new_bias [N]
// gets the q-th smallest (method 0) or its histogram estimate (method 1) of
// required = cutoff - z per expert.
hipError_t launch_qb_update(const float *logits, int64_t T, int N, int k, const float *bias, int q,
                            int method, float *req, float *new_bias, hipStream_t st);

// ---- router backward (route_bwd.hip) ---------------------------------------
// dz [T, N] from the logits, the forward's selection (idx, row_of), its
// expert outputs y_perm [R, d] and dy [T, d] (bf16); then dW_route [N, d]
// (through fp32 partials part [chunks][N][d]) and the router's du [T, d].
// aux_coef = aux_scale * alpha * N / T; stats[0..N) holds f.
int64_t route_bwd_chunks(int64_t T, int N, int d);
// d: width of u and W_route; dyw: width of dy and y_perm (d, or l).
hipError_t launch_route_backward(const float *logits, int64_t T, int N, int k, int d, int dyw,
                                 int renorm, const int32_t *idx, const int32_t *row_of,
                                 const float *y_perm, const uint16_t *dy, const float *stats,
                                 float aux_coef, const uint16_t *u, const uint16_t *w_route,
                                 float *part, float *dz, float *dw, float *du, hipStream_t st);

// ---- the experts' backward helpers (experts_bwd.hip) -------------------------
hipError_t launch_bwd_gather_dy(const uint16_t *dy, int64_t T, int d, int k,
                                const int32_t *row_of, const float *topk_w, uint16_t *dy_perm,
                                hipStream_t st);
hipError_t launch_transpose_bf16(const uint16_t *src, int B, int R, int C, uint16_t *dst,
                                 int64_t ld, int col0, hipStream_t st);
hipError_t launch_kseg(const int32_t *kept_offsets, int G, int32_t *kseg, hipStream_t st);
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st);
// dst [width][ld]: each expert's padded segment [kseg[g], kseg[g+1]) of the
// ld columns (ld a multiple of 64, >= kseg[G]) gets the expert's rows and
// zeros after them.
hipError_t launch_seg_transpose(const uint16_t *src, const uint16_t *src2, int64_t lds,
                                int width, const int32_t *kept_offsets,
                                const int32_t *offsets, const int32_t *perm, int kslots,
                                const int32_t *kseg, int G, int act, float bg, float bu,
                                uint16_t *dst, int64_t ld, hipStream_t st);
hipError_t launch_rows_sum(const float *rows, int64_t T, int d, int k, const int32_t *row_of,
                           float *dx, hipStream_t st);

// ---- the LatentMoE backward's per-token steps (latent_bwd.hip) --------------
// dr = RMSNorm backward at r = sum_kept a y_perm rows, given dn [T, width]
// fp32; writes dr and n = RMSNorm(r) as bf16 [T, width] (width <= 4096).
hipError_t launch_rms_backward(const float *y_perm, const int32_t *row_of, const float *topk_w,
                               int64_t T, int k, int width, float eps, const float *dn,
                               uint16_t *dr, uint16_t *n_out, hipStream_t st);
// n % 4 == 0 elements.
hipError_t launch_cast_bf16(const float *src, int64_t n, uint16_t *dst, hipStream_t st);
hipError_t launch_add_f32(float *dst, const float *src, int64_t n, hipStream_t st);
// Every token to each of S experts with weight 1: w [T*S], perm [S*T],
// row_of [T*S], offsets and kept_offsets [S+1].
hipError_t launch_shared_route(int64_t T, int S, float *w, int32_t *perm, int32_t *row_of,
                               int32_t *offsets, int32_t *kept_offsets, hipStream_t st);

// ---- decode-sized experts (decode.hip) -------------------------------------
// Max rows per expert the decode kernels take.
constexpr int kDecodeMaxRows = 64;
// The decode kernels read their activations (token rows) through a buffer
// resource of this many bytes from the matrix's start; the launchers refuse
// a matrix that does not fit it.
constexpr uint32_t kDecodeXBytes = 1u << 31;
// Routed-expert weight formats of the decode kernels (wfmt): bf16; E4M3
// codes with fp32 row scales s* ([N, h] gate/up, [N, w] down); MXFP4 (E2M1
// codes two a byte) with E8M0 block scales s* ([N, rows, K/32]).
enum WeightFormat { WFMT_BF16 = 0, WFMT_FP8 = 1, WFMT_MXFP4 = 2 };
hipError_t launch_decode_gu(const uint16_t *x, int64_t T, int w, const int32_t *perm,
                            const int32_t *offsets, const int32_t *kept_offsets, int kslots,
                            const void *Wg, const void *Wu, const void *sg, const void *su,
                            int wfmt, int h, int N, int act, float bg, float bu, uint16_t *hid,
                            hipStream_t st);
hipError_t launch_decode_down(const uint16_t *hid, int64_t T, const int32_t *kept_offsets,
                              const void *Wd, const void *sd, int wfmt, int h, int w, int N,
                              float *y_perm, hipStream_t st);

// ---- fp32 SIMT experts (simt.hip) ------------------------------------------
hipError_t launch_simt_gu(const float *x, const int32_t *perm, const int32_t *offsets,
                          const int32_t *kept_offsets, int kslots, const float *Wg,
                          const float *Wu, int w, int h, int N, int act, float bg, float bu,
                          float *hid, hipStream_t st);
hipError_t launch_simt_down(const float *hid, const int32_t *kept_offsets, const float *Wd,
                            int h, int w, int N, float *y_perm, hipStream_t st);

// ---- combine (combine.hip) ---------------------------------------------------
hipError_t launch_combine(const float *y_perm, const int32_t *row_of, const float *topk_w,
                          int64_t T, int k, int width, bool out_bf16, bool rmsnorm,
                          float eps, void *y, hipStream_t st);

}  // namespace moe

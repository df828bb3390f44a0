// Launchers implemented by the kernel translation units (included by common.h,
// after the argument structs). They validate nothing: the C-ABI layer checks
// every argument first. Each returns hipSuccess or the launch error.
#pragma once

hipError_t engram_launch_hash(const EngramHashArgs &a, const int32_t *token_map,
                              const int32_t *ids, int64_t batch, int64_t seq,
                              const int32_t *hist_in, int32_t *hist_out,
                              int64_t *row_ids, hipStream_t stream);

// Hash and gather of one Engram layer in one launch, one block per token, for
// decode-sized calls on an HBM-resident E4M3 table: the rows (bf16, [batch *
// seq, S * 256]) of the separate kernels, no row ids written. a.layers must be
// 1, and hist_out NULL or seq 1 (the history committed in place).
hipError_t engram_launch_hash_gather_e4m3(const EngramHashArgs &a, const int32_t *token_map,
                                          const int32_t *ids, int64_t batch, int64_t seq,
                                          const int32_t *hist_in, int32_t *hist_out,
                                          const uint8_t *table, int64_t table_rows,
                                          uint16_t *out, hipStream_t stream);
// The same rows split into codes [ntok * S, 256] and scales [ntok * S, 8], as
// engram_launch_gather_mx writes them.
hipError_t engram_launch_hash_gather_mx(const EngramHashArgs &a, const int32_t *token_map,
                                        const int32_t *ids, int64_t batch, int64_t seq,
                                        const int32_t *hist_in, int32_t *hist_out,
                                        const uint8_t *table, int64_t table_rows, uint8_t *codes,
                                        uint8_t *scales, hipStream_t stream);

// host_table: the table is pinned host memory; the gather then runs on a few
// CUs as a grid-strided kernel, leaving the rest to concurrent work.
hipError_t engram_launch_gather_e4m3(const uint8_t *table, int64_t table_rows,
                                     const int64_t *row_ids, int64_t n_ids,
                                     uint16_t *out, bool host_table, hipStream_t stream);

hipError_t engram_launch_gather_rows(const uint8_t *table, int64_t table_rows,
                                     const int64_t *row_ids, int64_t n_ids, uint8_t *out,
                                     bool host_table, hipStream_t stream);

// Rows split into their codes [n_ids, 256] and scales [n_ids, 8].
hipError_t engram_launch_gather_mx(const uint8_t *table, int64_t table_rows,
                                   const int64_t *row_ids, int64_t n_ids, uint8_t *codes,
                                   uint8_t *scales, bool host_table, hipStream_t stream);

hipError_t engram_launch_gather_f32(const float *table, int64_t table_rows,
                                    int32_t row_dim, const int64_t *row_ids,
                                    int64_t n_ids, float *out, hipStream_t stream);

// bf16 projection kv[m, n] = sum_k e[m, k] w[n, k]; w's rows are ldw >= k
// elements apart, e and kv are dense.
hipError_t engram_launch_gemm_bf16(const uint16_t *e, const uint16_t *w, int64_t ldw,
                                   uint16_t *kv, int64_t m, int64_t n, int64_t k, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream);

// The bf16 projection of hc keys and one value (n = (hc + 1) * dim, dim a
// multiple of 256) over 256 x 256 tiles whatever the token count: value columns
// stored as engram_launch_gemm_bf16's whole-tile kernel stores them, key tiles
// replaced by the gate's sums of each token (engram::gate_sums_pairs), which
// read h [m, hc * dim] and the folded gate weights qk_w [hc * dim].
hipError_t engram_launch_gemm_bf16_sums(const uint16_t *e, const uint16_t *w, int64_t ldw,
                                        const uint16_t *h, const float *qk_w, uint16_t *kv,
                                        int64_t m, int32_t hc, int32_t dim, int64_t k,
                                        hipStream_t stream);

// Whether engram_launch_gemm_bf16 runs this shape as whole 256 x 256 tiles
// (enough of them for every CU, no skinny decode schedule).
hipError_t engram_gemm_bf16_whole_tiles(int64_t m, int64_t n, int64_t k, bool *whole);

// Workspace the bf16 projection uses for a split-K schedule (0 when none).
hipError_t engram_gemm_bf16_workspace(int64_t m, int64_t n, int64_t k, size_t *bytes);

// Block-scaled FP8 projection: W codes [n, 256 S] and scales [n, 8 S], e the
// looked-up 264-byte rows [m, S, 264]; kv bf16 [m, n]. Split-K as for bf16
// when a large enough workspace is given.
hipError_t engram_launch_gemm_mx(const uint8_t *w_codes, const uint8_t *w_scales,
                                 const uint8_t *e_codes, const uint8_t *e_scales,
                                 int32_t segments, uint16_t *kv,
                                 int64_t m, int64_t n, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);
hipError_t engram_gemm_mx_workspace(int64_t m, int64_t n, int32_t segments, size_t *bytes);
// The block-scaled FP8 projection over whole 256 x 256 tiles with the gate's
// sums in the key tiles' epilogue (as engram_launch_gemm_bf16_sums), and
// whether engram_launch_gemm_mx runs a shape as whole tiles.
hipError_t engram_launch_gemm_mx_sums(const uint8_t *w_codes, const uint8_t *w_scales,
                                      const uint8_t *e_codes, const uint8_t *e_scales,
                                      int32_t segments, const uint16_t *h, const float *qk_w,
                                      uint16_t *kv, int64_t m, int32_t hc, int32_t dim,
                                      hipStream_t stream);
hipError_t engram_gemm_mx_whole_tiles(int64_t m, int64_t n, int32_t segments, bool *whole);

hipError_t engram_launch_gemm_f32(const float *e, const float *w, int64_t ldw, float *kv,
                                  int64_t m, int64_t n, int64_t k, hipStream_t stream);

// stats == NULL: the gate and the residual update. stats != NULL (float
// [tokens, hc + 1]): gates and the value row's mean square per token, h
// untouched. plain selects sigmoid(s) over the signed root. k_w == NULL: q_w
// holds the folded products q_w * k_w (engram_launch_fold_gate_weights).
hipError_t engram_launch_gate(bool f32, const int32_t *ids, EngramDeadRule dead_rule,
                              const void *kv, const float *q_w, const float *k_w,
                              void *h, float *gate_out, float *stats, int64_t tokens,
                              int32_t hc, int32_t dim, float eps, float clamp, int plain,
                              hipStream_t stream);

// The gate and residual update from the sums engram_launch_gemm_bf16_sums left
// in kv's key columns, the value row of kv and h (bf16; dim a multiple of 256).
// stats != NULL: engram_launch_gate's statistics mode on the sums instead.
hipError_t engram_launch_gate_sums(const int32_t *ids, EngramDeadRule dead_rule, const void *kv,
                                   void *h, float *gate_out, float *stats, int64_t tokens,
                                   int32_t hc, int32_t dim, float eps, float clamp, int plain,
                                   hipStream_t stream);

// qk_w[i] = q_w[i] * k_w[i] over hc * dim fp32 values (dim a multiple of 8).
hipError_t engram_launch_fold_gate_weights(const float *q_w, const float *k_w, float *qk_w,
                                           int32_t hc, int32_t dim, hipStream_t stream);

hipError_t engram_launch_short_conv(bool f32, const EngramConvArgs &c, const int32_t *ids,
                                    EngramDeadRule dead_rule, const void *kv, const float *stats,
                                    void *h, int64_t batch, int64_t seq, int32_t hc,
                                    int32_t dim, hipStream_t stream);

// dst[c * dst_ld + r] = src[r, c] for a row-major [rows, cols] array of 2- or
// 4-byte elements (layout.hip).
hipError_t engram_launch_transpose(const void *src, void *dst, int64_t rows, int64_t cols,
                                   int64_t dst_ld, int elem_bytes, hipStream_t stream);

/*
 * engram.h -- C ABI of the Engram conditional-memory layer forward for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (pages cited by title, then section / equation / table):
 *   [P1] "DeepSeek-V4.1 模型结构（5）：记忆，Engram"
 *   [P2] "Engram条件记忆：DeepSeek-V4.1-Flash中196B稀疏参数N-gram哈希查表的实现原理"
 *   [P3] "条件记忆：DeepSeek V4.1 Engram 如何用 O(1) 查表换掉一层计算"
 *   [P4] "ds4.c 学习笔记 · Engram"
 *   [P5] "DeepSeek Engram 详解：把静态知识从计算里拆出来"
 *
 *   1. x' = P(x): raw token id -> compressed id ([P1] "tokenizer 压缩").
 *   2. mix_{t,n} = XOR_{i<n} x'_{t-i} m_i; row_{t,n,k} = (mix mod p_{n,k}) + off_{n,k}
 *      ([P1] eq. (H) and "一层只有一张表").
 *   3. Gather the S = (N-1) K rows of 264 bytes (256 E4M3 + 8 E8M0 scales, one
 *      scale per 32 values) and dequantise them to bf16 ([P4] "布局与哈希探测";
 *      [P1] "196B 参数怎么存、怎么取").
 *   4. kv = e W: hc keys and one value in one projection ([P1] "每条流一个 key
 *      的设计沿用自原版"; [P5] §4.3).
 *   5. Per stream m: s = RMSNorm(h_m) . RMSNorm(k_m) / sqrt(d) with the learned
 *      scales q_w * k_w, alpha = sigmoid(sign(s) sqrt(max(|s|, clamp))),
 *      h_m <- bf16(h_m + alpha v); alpha = 0 and h untouched at DEAD positions
 *      ([P1] "门控", "sigmoid 之前多一步带符号的平方根"; [P4] "消费：学习投影 +
 *      余弦门控").
 *   Variants the papers describe: the plain gate alpha = sigmoid(s) ([P5] §4.1;
 *   engram_forward_desc.gate_mode) and the short convolution branch after the
 *   gate, Y = SiLU(Conv1D(RMSNorm(alpha v))) + alpha v, h_m += Y ([P5] §4.2;
 *   [P3] §三; engram_gate_conv, engram_forward_conv).
 *
 * Conventions for every entry point:
 *   - Pointers are device memory unless marked [host]. The caller owns every
 *     buffer; the library allocates nothing, keeps no state between calls
 *     (beyond a per-thread record of the last HIP error) and never
 *     synchronises: work is enqueued on `stream` (0 = null stream) and
 *     completes asynchronously.
 *   - All arrays are dense row-major. Device pointers must be 16-byte aligned.
 *   - Arguments are validated on the host before any launch; a failed check
 *     returns a negative engram_status and enqueues nothing. A failed launch
 *     returns ENGRAM_EHIP; engram_last_hip_error names the HIP error behind it.
 *   - Device data cannot be validated synchronously, so it follows conventions:
 *     a raw id outside [0, V) (the DEAD marker -1 included), or one the token
 *     map sends outside [0, V'), is a DEAD cell; a history entry outside
 *     [0, V') is DEAD; a row id outside [0, rows) gathers a zero row ([P3] §五:
 *     out-of-range rows output zero rows). The gate decides DEAD positions from
 *     the raw id alone, so a map must pass engram_check_token_map first.
 *   - Calls that write overlapping buffers on different streams race.
 *
 * Host-resident tables ([P1] "放在第 1 层和第 14 层", last paragraph: the rows a
 * step needs depend on the token ids alone, so the table can stay in host memory
 * and the rows move to the GPU while earlier layers compute; [P5] §8.2-§8.4:
 * prefetch on a separate path, wait for its completion event, stall =
 * max(0, T_fetch - T_window); [P3] §五: the host link's bandwidth is the cost).
 * Every entry point that reads a table (engram_gather, engram_gather_rows,
 * engram_gather_mx, engram_forward, engram_forward_conv, engram_forward_mx)
 * accepts pinned host memory (hipHostMalloc, or torch's pin_memory) as well as
 * device memory: its kernels then read the 264-byte rows over the host link
 * themselves, straight into HBM, with no staging copy on the host. A prefetch is
 * engram_hash + engram_gather (or engram_gather_mx) on a second stream, ordered
 * before the consuming engram_project (or engram_project_mx) by an event. A table
 * pointer the device cannot read (pageable host memory, an unknown address) is
 * rejected with ENGRAM_EINVAL before any launch.
 */
#ifndef ENGRAM_H
#define ENGRAM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ENGRAM_DEAD (-1)
#define ENGRAM_MAX_NGRAM 8        /* N, largest n-gram order (orders 2..N) */
#define ENGRAM_MAX_SEGMENTS 64    /* S = (N - 1) * K */
#define ENGRAM_MAX_LAYERS 4       /* Engram layers hashed in one engram_hash_layers call */
#define ENGRAM_MAX_TOTAL_SEGMENTS 128  /* layers * S in one engram_hash_layers call */
#define ENGRAM_ROW_BYTES 264      /* E4M3 row: 256 payload bytes + 8 scale bytes */
#define ENGRAM_ROW_DIM_E4M3 256
#define ENGRAM_MAX_CONV_TAPS 8    /* kernel size w of the short convolution */
#define ENGRAM_MAX_CONV_HISTORY 64 /* (w - 1) * dilation */
/* Scratch array of engram_forward_static, per GPU: 64 MiB, enough for a decode
 * step of up to 1024 tokens at hc 4 x 5120 with 24 segments. */
#define ENGRAM_STATIC_SCRATCH_BYTES (64ull << 20)

typedef enum engram_status {
  ENGRAM_OK = 0,
  ENGRAM_EINVAL = -1,     /* null / misaligned pointer, negative size, bad enum  */
  ENGRAM_EVOCAB = -2,     /* compressed vocabulary does not match the token map  */
  ENGRAM_EMULT = -3,      /* multiplier even, < 1 or > floor((2^63-1)/V')         */
  ENGRAM_ESHAPE = -4,     /* inconsistent shapes                                  */
  ENGRAM_EWORKSPACE = -5, /* workspace missing or too small                       */
  ENGRAM_EHIP = -6,       /* a HIP launch failed                                  */
  ENGRAM_EPRIMES = -7,    /* prime < 2 or >= 2^32, offsets not the prefix sums,
                             or rows beyond the table                             */
  ENGRAM_ESCRATCH = -8    /* engram_forward_static: the call needs more scratch
                             than ENGRAM_STATIC_SCRATCH_BYTES                     */
} engram_status;

typedef enum engram_row_format {
  ENGRAM_ROW_E4M3_E8M0_264 = 0, /* uint8 [rows, 264]: 256 E4M3FN bytes in element
                                   order, then 8 E8M0 scales; value =
                                   E4M3(q_c) * 2^(s_{c/32} - 127), emitted as bf16 */
  ENGRAM_ROW_F32 = 1            /* float [rows, row_dim], copied verbatim          */
} engram_row_format;

/*
 * Hash setup of one Engram layer ([P1] eq. (H); [P2] config.json table;
 * [P3] §2.2, §4.3). Passed by pointer, read on the host at call time; the
 * numeric fields travel to the kernels by value.
 */
typedef struct engram_hash_params {
  int32_t raw_vocab;          /* V (129280)                                        */
  int32_t compressed_vocab;   /* V' (99092): the vocabulary the multipliers are
                                 bounded for ([P1] §"哈希函数", item on overflow)   */
  int32_t max_ngram;          /* N, orders 2..N; 2 <= N <= ENGRAM_MAX_NGRAM (4)    */
  int32_t heads;              /* K heads per order (8); S = (N-1) K segments       */
  int32_t pad_id;             /* compressed pad id, in [0, V')                     */
  int32_t reserved;           /* must be 0                                         */
  const int32_t *token_map;   /* device [V], values in [0, V'); validate once with
                                 engram_check_token_map                            */
  int64_t multipliers[ENGRAM_MAX_NGRAM]; /* m_0..m_{N-1}; m_i multiplies the token
                                 i positions back; odd, 1 <= m <= (2^63-1)/V'      */
  int64_t primes[ENGRAM_MAX_SEGMENTS];   /* p_j of segment j = (n-2) K + k,
                                 2 <= p_j < 2^32                                   */
  int64_t offsets[ENGRAM_MAX_SEGMENTS];  /* off_j = p_0 + ... + p_{j-1}            */
} engram_hash_params;

typedef enum engram_gate_mode {
  ENGRAM_GATE_SIGNED_SQRT = 0, /* sigmoid(sign(s) sqrt(max(|s|, clamp))): the released
                                  code's gate ([P1] "sigmoid 之前多一步带符号的平方根") */
  ENGRAM_GATE_PLAIN = 1        /* sigmoid(s): the papers' own formula ([P5] §4.1);
                                  gate_clamp is ignored                             */
} engram_gate_mode;

/* Shapes and constants of one forward call. */
typedef struct engram_forward_desc {
  int64_t batch;              /* B sequences                                       */
  int64_t seq;                /* T tokens per sequence in this chunk (decode: 1);
                                 B, T >= 0 and B * T <= 2^31 - 1, else ESHAPE      */
  int32_t hc;                 /* hyper-connection streams (4); 1 <= hc <= 8        */
  int32_t dim;                /* d, stream width (5120); multiple of 8             */
  int64_t table_rows;         /* R, rows of the table; >= sum of the primes        */
  int32_t row_format;         /* engram_row_format                                 */
  int32_t row_dim;            /* 256 for E4M3 rows; multiple of 4 for fp32 rows    */
  float eps;                  /* RMS epsilon (1e-6)                                */
  float gate_clamp;           /* c in sqrt(max(|s|, c)) (0)                        */
  int32_t gate_mode;          /* engram_gate_mode (ENGRAM_GATE_SIGNED_SQRT)         */
  int32_t wkv_ld;             /* elements between consecutive wkv rows; 0 = dense
                                 (S row_dim). See engram_project. Ignored by the
                                 entry points that take no wkv                     */
} engram_forward_desc;

/*
 * The short convolution branch after the gate ([P5] §4.2: depthwise, causal,
 * kernel size 4 at dilation 3 = the largest n-gram order, so position t reads
 * t, t-3, t-6, t-9; RMSNorm before and SiLU after; filters start at zero, which
 * makes the branch's output the gated value itself; [P5] §9.5: decode and
 * chunked prefill keep the last 9 positions). For stream m, channel c:
 *   V~_t = alpha_{t,m} v_t,  n_t = V~_t / sqrt(mean_c(V~_t^2) + eps) * norm_weight[m][c],
 *   u_t = sum_j weight[m][c][j] * n_{t - (w-1-j) dilation},  (n = 0 before the
 *   sequence start when there is no history)
 *   h_{t,m,c} <- round(h + SiLU(u_t) + V~_t),  except at DEAD positions, whose
 *   streams stay untouched and whose V~ is 0 for the positions after them.
 * History of a sequence, L = (w - 1) * dilation positions before the chunk, in
 * factored form: state_v [B, L, dim] holds their value rows v (kv's dtype:
 * bf16, or float for ENGRAM_ROW_F32) and state_s float [B, L, hc + 1] their
 * gates alpha_0..alpha_{hc-1} and mean(v^2); a DEAD or pre-start position has
 * alpha = 0. Zeroed buffers are the history of a sequence start.
 */
typedef struct engram_short_conv {
  int32_t taps;               /* w (4); 1 <= w <= ENGRAM_MAX_CONV_TAPS             */
  int32_t dilation;           /* (3); >= 1, (w - 1) * dilation <= ENGRAM_MAX_CONV_HISTORY */
  float eps;                  /* RMSNorm epsilon of the branch, > 0                */
  int32_t reserved;           /* must be 0                                         */
  const float *weight;        /* device float [hc, dim, w]; zeros = the papers' init */
  const float *norm_weight;   /* device float [hc, dim], or NULL for ones          */
  const void *state_v_in;     /* device history before the chunk, or NULL for a    */
  const float *state_s_in;    /*   sequence start (both NULL or both set)          */
  void *state_v_out;          /* device history after the chunk, or NULL to skip   */
  float *state_s_out;         /*   (both NULL or both set); may equal the inputs   */
} engram_short_conv;

/* Message for a status code (static storage). */
const char *engram_status_string(int status);

/* hipGetErrorString of the HIP error behind the last ENGRAM_EHIP an entry
 * point returned on the calling host thread ("no error" if none). This record
 * is the library's only state; it is per thread and never cleared. */
const char *engram_last_hip_error(void);

/* sizeof the two structs as this library was built, for bindings to check. */
size_t engram_sizeof_hash_params(void);
size_t engram_sizeof_forward_desc(void);
size_t engram_sizeof_short_conv(void);

/*
 * [host] Segment sizes and offsets: the first `count` primes >= base, in
 * ascending order, one per segment and never reused, and their exclusive
 * prefix sums ([P1] "一层只有一张表": the row count is the sum of the 24
 * primes found upward from 16,000,000). Deterministic Miller-Rabin.
 * primes_out, offsets_out: [host] int64 [count]; total_rows_out: [host] or NULL.
 * Errors: ENGRAM_EINVAL (count < 0, null, base < 2 or a prime >= 2^32).
 */
int engram_make_primes(int64_t base, int32_t count, int64_t *primes_out,
                       int64_t *offsets_out, int64_t *total_rows_out);

/*
 * [host] Tables of several Engram layers: the first layers * per_layer primes
 * >= base, ascending and never reused, dealt to the layers in order (layer l
 * takes primes [l * per_layer, (l + 1) * per_layer)); each layer has its own
 * table, so offsets restart at 0 in every layer and rows_out[l] is the sum of
 * layer l's primes ([P1] "一层只有一张表" and its table of the two layers:
 * 16000057..16000463, sum 384006168, then 16000477..16000889, sum 384016682;
 * [P3] §2.2: primes drawn in (layer, order, head) order).
 * primes_out, offsets_out: [host] int64 [layers * per_layer], layer-major;
 * rows_out: [host] int64 [layers] or NULL.
 * Errors: ENGRAM_EINVAL (layers < 1, per_layer < 0, null, base < 2 or a prime
 * >= 2^32).
 */
int engram_make_layer_primes(int64_t base, int32_t layers, int32_t per_layer,
                             int64_t *primes_out, int64_t *offsets_out, int64_t *rows_out);

/*
 * [host] Start-up check that the compression map matches the configured
 * compressed vocabulary: every value in [0, V'), every compressed id used, and
 * so max + 1 == V' ([P1] §"哈希函数": a mismatch means every row id is wrong;
 * [P3] §2.1). token_map: [host] int32 [raw_vocab].
 * Errors: ENGRAM_EINVAL, ENGRAM_EVOCAB.
 */
int engram_check_token_map(const int32_t *token_map, int32_t raw_vocab,
                           int32_t compressed_vocab);

/*
 * Steps 1-2: row ids of every (position, segment).
 *   ids      int32 [B, T] raw ids, -1 = DEAD (image or padding position)
 *   hist_in  int32 [B, N-1] or NULL. The N-1 cells before this chunk, oldest
 *            first: compressed ids or -1 (DEAD). NULL = sequence start: those
 *            cells are the pad id, looked up like any id ([P1] §"哈希函数";
 *            [P4] "布局与哈希探测": the hash state is the tail of 3 tokens).
 *   hist_out int32 [B, N-1] or NULL. State after the chunk: the last N-1
 *            positions' compressed ids (-1 at DEAD), older slots shifted in from
 *            hist_in (or the pad id). May alias hist_in.
 *   row_ids  int64 [B*T, S], row_ids[t, (n-2) K + k] = (mix_{t,n} mod p) + off.
 * A DEAD cell blocks itself and every older cell, which then hash as the pad id;
 * at a DEAD position every cell is blocked ([P1] image-token paragraph; [P2]
 * "多模态细节"; [P4] item 4). B or T may be 0; B * T above 64 * (2^31 - 1)
 * is ENGRAM_ESHAPE.
 * Errors: ENGRAM_EINVAL, ENGRAM_EMULT, ENGRAM_EPRIMES, ENGRAM_ESHAPE, ENGRAM_EHIP.
 */
int engram_hash(const engram_hash_params *params, const int32_t *ids, int64_t batch,
                int64_t seq, const int32_t *hist_in, int32_t *hist_out,
                int64_t *row_ids, hipStream_t stream);

/*
 * Steps 1-2 for several Engram layers over the same tokens, in one pass: the
 * cells (and the history) are built once, then each layer mixes them with its
 * own multipliers and reduces them modulo its own primes ([P1] "一层只有一张表":
 * the layers' primes and multipliers are drawn independently, so an n-gram
 * lands on unrelated rows; [P3] §2.4: every layer's row ids depend on the
 * token ids only and are computed before the layer loop).
 *   params   [host] engram_hash_params [layers]. All layers share raw_vocab,
 *            compressed_vocab, max_ngram, heads, pad_id and token_map; each
 *            has its own multipliers, primes and offsets (offsets of its own
 *            table, see engram_make_layer_primes).
 *   layers   1 <= layers <= ENGRAM_MAX_LAYERS, layers * S <= ENGRAM_MAX_TOTAL_SEGMENTS.
 *   row_ids  int64 [layers, B*T, S]: layer l's ids are the contiguous slice
 *            row_ids + l * B*T*S, ready for that layer's engram_gather.
 *   ids, hist_in, hist_out as for engram_hash (the history has no layer).
 * With layers = 1 this is engram_hash.
 * Errors: ENGRAM_EINVAL (also: the layers disagree on a shared field),
 * ENGRAM_EMULT, ENGRAM_EPRIMES, ENGRAM_ESHAPE, ENGRAM_EHIP.
 */
int engram_hash_layers(const engram_hash_params *params, int32_t layers, const int32_t *ids,
                       int64_t batch, int64_t seq, const int32_t *hist_in, int32_t *hist_out,
                       int64_t *row_ids, hipStream_t stream);

/*
 * Step 3: gather and dequantise rows ([P3] §2.3: fp8 E4M3 payload and E8M0
 * block scales, bf16 output; [P4] "永不常驻的 I/O 设计": 32 values share a scale).
 *   table    row_format rows: uint8 [table_rows, 264] or float [table_rows, row_dim],
 *            in device memory or in pinned host memory (see "Host-resident tables")
 *   row_ids  int64 [n_ids]; ids outside [0, table_rows) give zero rows
 *   out      [n_ids, row_dim] bf16 (E4M3 rows, row_dim = 256) or float (fp32 rows)
 * Dequantisation is exact: E4M3(q) * 2^(s - 127) rounded once to bf16 (nearest,
 * ties to even; NaN codes and scale 0xFF give NaN).
 * Errors: ENGRAM_EINVAL, ENGRAM_ESHAPE, ENGRAM_EHIP.
 */
int engram_gather(const void *table, int64_t table_rows, int32_t row_format,
                  int32_t row_dim, const int64_t *row_ids, int64_t n_ids, void *out,
                  hipStream_t stream);

/*
 * Step 3 without dequantisation: the looked-up rows, bytes unchanged (256 E4M3
 * codes then 8 E8M0 scales each; [P4] "永不常驻的 I/O 设计"). A row id outside
 * [0, table_rows) gives a zero row ([P3] §五).
 *   table    uint8 [table_rows, 264], 8-byte aligned, in device memory or in pinned
 *            host memory (see "Host-resident tables")
 *   row_ids  int64 [n_ids]
 *   out      uint8 [n_ids, 264], 8-byte aligned
 * Errors: ENGRAM_EINVAL, ENGRAM_ESHAPE, ENGRAM_EHIP.
 */
int engram_gather_rows(const void *table, int64_t table_rows, const int64_t *row_ids,
                       int64_t n_ids, void *out, hipStream_t stream);

/*
 * Step 3 for engram_project_mx: the looked-up rows split into their codes and
 * their scales (bytes unchanged), so that the S rows of a token form one
 * K = 256 S long row of E4M3 inputs with K/32 E8M0 block scales, the layout of
 * the FP8 weight. A row id outside [0, table_rows) gives zero codes and scales.
 *   table    as engram_gather_rows
 *   row_ids  int64 [n_ids]
 *   codes    uint8 [n_ids, 256], 16-byte aligned
 *   scales   uint8 [n_ids, 8], 8-byte aligned
 * Errors: ENGRAM_EINVAL, ENGRAM_ESHAPE, ENGRAM_EHIP.
 */
int engram_gather_mx(const void *table, int64_t table_rows, const int64_t *row_ids,
                     int64_t n_ids, void *codes, void *scales, hipStream_t stream);

/*
 * Step 4: kv = e W ([P1] "每条流一个 key 的设计沿用自原版": one 6144 x 25600
 * matrix; [P4] "消费": the weight is stored with the 6144 inputs innermost).
 *   e    [tokens, in_dim]       bf16 (act_f32 = 0) or float (act_f32 = 1)
 *   wkv  [out_dim, in_dim]      same type; row c holds the weights of output c
 *                               and starts wkv_ld elements after row c - 1; the
 *                               buffer holds at least (out_dim - 1) wkv_ld +
 *                               in_dim elements (the gaps are never read)
 *   wkv_ld                      0 (= in_dim, dense rows), or >= in_dim and a
 *                               multiple of 16 bytes, at most 2^20 for bf16.
 *                               The results do not depend on it. Rows a
 *                               multiple of 4 KiB apart (in_dim 6144 bf16)
 *                               put every CU's loads of one K-step at the same
 *                               offset within a memory page, which costs a
 *                               call that streams the weight from HBM once
 *                               (<= 256 tokens) about 10 %;
 *                               engram_wkv_row_stride gives a stride that avoids it
 *   kv   [tokens, out_dim]      same type; fp32 accumulation, bf16 rounded to
 *                               nearest-even
 *   workspace, workspace_bytes
 *        NULL, or at least engram_project_workspace_size bytes, 256-byte
 *        aligned. A bf16 call of at most 256 tokens with 64-128 output columns
 *        per CU and in_dim % 384 == 0 (decode) deals columns to the CUs and
 *        needs none. Other calls with fewer 256 x 256 output tiles than the GPU
 *        has CUs split K over the CUs and keep fp32 partial tiles here, summed
 *        afterwards in a fixed order (the result depends only on the shape and
 *        the CU count); with NULL they use narrower tiles over the whole K.
 *        Every other path sums each output's K in one order, so its bits do
 *        not depend on the token count. Contents need not be initialised and
 *        are clobbered.
 * bf16 requires in_dim % 64 == 0, out_dim % 8 == 0, in_dim <= 2^20 and
 * ceil(tokens / 256) * ceil(out_dim / 128) < 2^23 (the kernels address a
 * 256-row operand panel with 32-bit byte counts and launch at most 2^32
 * threads); fp32 requires in_dim % 4 == 0 and out_dim % 4 == 0. The same tile
 * bound applies to engram_project_mx and to the forward entry points.
 * Errors: ENGRAM_EINVAL, ENGRAM_ESHAPE (also a wkv_ld outside the rule above),
 * ENGRAM_EWORKSPACE (non-NULL and too small or misaligned), ENGRAM_EHIP.
 */
int engram_project(const void *e, const void *wkv, void *kv, int64_t tokens,
                   int64_t in_dim, int64_t out_dim, int64_t wkv_ld, int32_t act_f32,
                   void *workspace, size_t workspace_bytes, hipStream_t stream);

/* [host] A wkv row stride for engram_project and engram_forward_desc.wkv_ld:
 * in_dim rounded up to 128 bytes, plus 128 bytes when that is a multiple of
 * 4 KiB (6144 bf16 -> 6208). 0 for in_dim outside [1, 2^20] or elem_bytes not 2
 * or 4. */
int64_t engram_wkv_row_stride(int64_t in_dim, int32_t elem_bytes);

/* [host] Bytes of workspace engram_project uses for these sizes on the current
 * device (0 if it needs none, on bad arguments or on a HIP error). */
size_t engram_project_workspace_size(int64_t tokens, int64_t in_dim, int64_t out_dim,
                                     int32_t act_f32);

/*
 * Step 4 with a block-scaled FP8 weight ([P3] §2.3: the projection weight is
 * block-FP8 beside the fp8 e4m3 + e8m0 table; [P5] §4.3: the projections fuse
 * into one dense FP8 matrix product). Reading: the weight uses the table's own
 * block encoding, E4M3 values with one E8M0 scale per 32 consecutive inputs.
 * kv[t, c] = sum_k e[t, k] W[c, k] with e[t, 256 j + i] = E4M3(row_j[i]) *
 * 2^(row_j[256 + i / 32] - 127) taken straight from the looked-up rows' codes
 * and scales (exact products, fp32 accumulation in gfx950's block-scaled FP8
 * MFMA), rounded once to bf16 nearest-even.
 *   e_codes  uint8 [tokens, 256 segments], 16-byte aligned: engram_gather_mx codes
 *   e_scales uint8 [tokens, 8 segments], 4-byte aligned: engram_gather_mx scales
 *   w_codes  uint8 [out_dim, 256 segments], 16-byte aligned
 *   w_scales uint8 [out_dim, 8 segments] (E8M0, bias 127), 4-byte aligned
 *   kv       bf16 [tokens, out_dim]; out_dim % 8 == 0
 *   workspace as for engram_project, sized by engram_project_mx_workspace_size
 * Errors: ENGRAM_EINVAL, ENGRAM_ESHAPE, ENGRAM_EWORKSPACE, ENGRAM_EHIP.
 */
int engram_project_mx(const void *e_codes, const void *e_scales, int32_t segments,
                      const void *w_codes, const void *w_scales, void *kv, int64_t tokens,
                      int64_t out_dim, void *workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * Re-layout of a caller's weight buffer, once, outside the per-step path:
 * dst[c * dst_ld + r] = src[r, c] for a row-major [rows, cols] array of 2-byte
 * (bf16) or 4-byte (fp32) elements; dst_ld = 0 means rows (dense). The kernels read wkv as [(hc+1) dim, S row_dim]
 * (inputs innermost, [P4] "消费") and the gate scales as [hc, dim]. A caller
 * holding them the other way round, wkv as [S row_dim, (hc+1) dim] (the
 * 6144 x 25600 matrix of [P1] "每条流一个 key 的设计沿用自原版" with outputs
 * innermost) or q_w / k_w as [dim, hc], calls
 *   engram_transpose(wkv_in_out, wkv, S row_dim, (hc+1) dim, wkv_ld, 2 or 4, stream)
 *   engram_transpose(q_w_dim_hc, q_w, dim, hc, 0, 4, stream)
 * and passes the results to every entry point (wkv_ld as engram_project's, 0
 * for dense rows); the forward's bits are those of the same weights stored in
 * the kernels' layout.
 *   src, dst  device, elem_bytes-aligned, caller-owned, not overlapping; dst
 *             holds (cols - 1) dst_ld + rows elements, the gaps untouched
 * Errors: ENGRAM_EINVAL (elem_bytes not 2 or 4, null, misaligned or
 * overlapping buffers), ENGRAM_ESHAPE (negative sizes, 0 < dst_ld < rows, or
 * more than 2^24 tiles of 64 x 64), ENGRAM_EHIP.
 */
int engram_transpose(const void *src, void *dst, int64_t rows, int64_t cols, int64_t dst_ld,
                     int32_t elem_bytes, hipStream_t stream);

/* [host] Bytes of workspace engram_project_mx uses (0 if none, on bad arguments
 * or on a HIP error). */
size_t engram_project_mx_workspace_size(int64_t tokens, int32_t segments, int64_t out_dim);

/*
 * Step 5: gate and residual update, given kv.
 *   desc     shapes (batch, seq, hc, dim, row_format selects bf16 or fp32 I/O,
 *            eps, gate_clamp); table fields are ignored
 *   ids      int32 [B, T] raw ids; a position with an id outside [0, raw_vocab)
 *            is DEAD: alpha = 0 and its h is left untouched. (The fused entry
 *            points, engram_forward and its variants, also make a position DEAD
 *            whose token map value lies outside [0, compressed_vocab), as the
 *            hash does, so gate and row ids agree even for a map that would
 *            fail engram_check_token_map.)
 *   kv       [B*T, (hc+1) dim]: keys k^(0..hc-1) then the value v
 *   q_w, k_w float [hc, dim]: learned scales of stream m in row m
 *   h        [B, T, hc, dim] in/out, bf16 (E4M3 format) or float (fp32 format)
 *   gate_out float [B*T, hc] or NULL
 * Errors: ENGRAM_EINVAL, ENGRAM_ESHAPE, ENGRAM_EHIP.
 */
int engram_gate(const engram_forward_desc *desc, const int32_t *ids, int32_t raw_vocab,
                const void *kv, const float *q_w, const float *k_w, void *h,
                float *gate_out, hipStream_t stream);

/*
 * The two learned scales enter the gate only through their element-wise
 * product ([P4] "消费：学习投影 + 余弦门控": the dot weights element i of h and
 * k by q_w[i] k_w[i]), so they can be folded once into one array.
 *   q_w, k_w float [hc, dim] device, 16-byte aligned, dim a multiple of 8
 *   qk_w     float [hc, dim] device, 16-byte aligned, caller-owned:
 *            qk_w[i] = q_w[i] * k_w[i] (one fp32 rounding, the product the
 *            gate forms itself), so engram_gate_folded gives engram_gate's bits
 * Errors: ENGRAM_EINVAL, ENGRAM_ESHAPE, ENGRAM_EHIP.
 */
int engram_fold_gate_weights(const float *q_w, const float *k_w, int32_t hc, int32_t dim,
                             float *qk_w, hipStream_t stream);

/*
 * Step 5 with folded scales: engram_gate with qk_w (from engram_fold_gate_weights)
 * in place of q_w and k_w. It reads one scale array per stream instead of two.
 * Arguments and errors as engram_gate.
 */
int engram_gate_folded(const engram_forward_desc *desc, const int32_t *ids, int32_t raw_vocab,
                       const void *kv, const float *qk_w, void *h, float *gate_out,
                       hipStream_t stream);

/*
 * Steps 4 and 5 with the key side of the gate in the projection's epilogue
 * ([P3] §2.3, the context gate fused with the single projection; [P1] "门控"
 * and [P4] "消费：学习投影 + 余弦门控" for the sums). The gate of stream m
 * needs of its keys only sum_i k_i^2 and sum_i h_i q_w,i k_w,i k_i, so the
 * projection forms them per 128-column block while the keys are still in
 * registers, and no key is written to memory. engram_forward takes this path
 * whenever the projection fills the CUs with whole 256 x 256 tiles (bf16 rows,
 * dim % 256 == 0); these two entry points are its launches, for tests and
 * timing (engram_forward_conv: engram_gate_conv_sums in place of
 * engram_gate_sums).
 *
 * engram_project_gate_sums: kv = e W over 256 x 256 tiles, whatever the token
 * count.
 *   desc     batch * seq tokens, hc, dim (a multiple of 256), wkv_ld; row_format
 *            must be ENGRAM_ROW_E4M3_E8M0_264 (bf16 activations)
 *   e, in_dim, wkv   as engram_project (bf16; in_dim % 64 == 0)
 *   h        [tokens, hc, dim] bf16, the streams the gate will update (read only)
 *   qk_w     [hc, dim] float, q_w * k_w (engram_fold_gate_weights)
 *   kv       [tokens, (hc+1) dim] bf16. The value columns [hc dim, (hc+1) dim)
 *            get engram_project's bits for a call that fills the CUs with whole
 *            tiles (every call of this entry point sums each output's K in that
 *            order). The first hc * dim / 128 float pairs of each row (8-byte
 *            aligned, inside its key columns) get, for stream m and column block
 *            b, pair m * (dim / 128) + b = (sum k^2, sum h q_w k_w k) over
 *            columns [128 b, 128 b + 128) of that stream, k rounded to bf16 as
 *            engram_project would store it, fp32 sums. The other key columns
 *            are not written.
 * Errors: ENGRAM_EINVAL (NULL or misaligned pointers, fp32 rows),
 * ENGRAM_ESHAPE (dim % 256, in_dim, wkv_ld or the tile bound of
 * engram_project), ENGRAM_EHIP.
 *
 * engram_gate_sums: step 5 from those sums, the value columns of kv and h.
 *   desc, ids, raw_vocab, h, gate_out   as engram_gate (bf16 rows, dim % 256 == 0)
 *   kv       as left by engram_project_gate_sums
 * The gates equal engram_gate's on the same keys up to the order of the fp32
 * sums. Errors as engram_gate, and ENGRAM_EINVAL for fp32 rows.
 */
int engram_project_gate_sums(const engram_forward_desc *desc, const void *e, int64_t in_dim,
                             const void *wkv, const void *h, const float *qk_w, void *kv,
                             hipStream_t stream);
int engram_gate_sums(const engram_forward_desc *desc, const int32_t *ids, int32_t raw_vocab,
                     const void *kv, void *h, float *gate_out, hipStream_t stream);

/*
 * engram_gate_conv from the sums of engram_project_gate_sums: the gate's
 * statistics (gates and the value row's mean square per token) from the sums,
 * the value columns of kv and h, then the short convolution branch as in
 * engram_gate_conv. engram_forward_conv takes this path under the rule of
 * engram_forward. Arguments and errors as engram_gate_conv without q_w and k_w
 * (they are inside the sums), bf16 rows and dim % 256 == 0 only
 * (ENGRAM_EINVAL, ENGRAM_ESHAPE).
 */
int engram_gate_conv_sums(const engram_forward_desc *desc, const engram_short_conv *conv,
                          const int32_t *ids, int32_t raw_vocab, const void *kv, void *h,
                          float *gate_out, void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * engram_project_gate_sums for the block-scaled FP8 weight: engram_project_mx's
 * operands (e_codes, e_scales, segments, w_codes, w_scales as there) over whole
 * 256 x 256 tiles, h and qk_w as engram_project_gate_sums, kv laid out as
 * there (value columns with engram_project_mx's whole-tile bits, the sums in
 * the key columns). engram_forward_mx takes this path under the same rule as
 * engram_forward. Errors as engram_project_mx, and ENGRAM_ESHAPE for
 * dim % 256 != 0.
 */
int engram_project_mx_gate_sums(const engram_forward_desc *desc, const void *e_codes,
                                const void *e_scales, int32_t segments, const void *w_codes,
                                const void *w_scales, const void *h, const float *qk_w,
                                void *kv, hipStream_t stream);

/* Bytes of workspace engram_forward needs (row ids, e, kv, the folded gate
 * scales and the projection's workspace), or 0 on bad args. Calls of 2048
 * tokens or more fold q_w * k_w there (engram_fold_gate_weights; the same
 * bits), so the gate reads one scale array per stream. */
size_t engram_forward_workspace_size(const engram_hash_params *params,
                                     const engram_forward_desc *desc);

/*
 * Steps 1-5 for one chunk of B sequences x T tokens, on one stream.
 *   ids, hist_in, hist_out   as engram_hash
 *   table                    as engram_gather, desc->row_format / row_dim
 *   wkv                      [(hc+1) dim, S row_dim], bf16 (E4M3) or float (fp32),
 *                            rows desc->wkv_ld elements apart (engram_project)
 *   q_w, k_w, h, gate_out    as engram_gate
 *   workspace                device, >= engram_forward_workspace_size bytes,
 *                            256-byte aligned; contents are scratch
 * Errors: any of the stage errors, ENGRAM_EWORKSPACE.
 */
int engram_forward(const engram_hash_params *params, const engram_forward_desc *desc,
                   const int32_t *ids, const int32_t *hist_in, int32_t *hist_out,
                   const void *table, const void *wkv, const float *q_w,
                   const float *k_w, void *h, float *gate_out, void *workspace,
                   size_t workspace_bytes, hipStream_t stream);

/*
 * engram_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). It makes engram_forward's launches, taking their
 * scratch (row ids, e, kv, folded gate scales) from a static device array of
 * ENGRAM_STATIC_SCRATCH_BYTES that every GPU the library runs on holds until
 * the process ends. The call itself allocates nothing. Its results are
 * engram_forward's bits, except where engram_forward would split the
 * projection's K over the CUs (more than 256 tokens but fewer 256 x 256 tiles
 * than CUs): those partial tiles do not fit, so the projection runs 128-wide
 * tiles over the whole K instead (the bits of a call with many tokens), which
 * can differ from the split sum in the last bits of kv.
 *   arguments as engram_forward, without workspace / workspace_bytes
 *   stream    must belong to the current device
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (two streams, two host threads)
 * race. Nothing in the array needs to start at zero.
 * Errors: as engram_forward; ENGRAM_ESCRATCH when the row ids, e, kv and folded
 * scales of the call (engram_forward_workspace_size without the projection's
 * part) exceed ENGRAM_STATIC_SCRATCH_BYTES (checked before any launch);
 * ENGRAM_EINVAL when the stream is not on the current device.
 */
int engram_forward_static(const engram_hash_params *params, const engram_forward_desc *desc,
                          const int32_t *ids, const int32_t *hist_in, int32_t *hist_out,
                          const void *table, const void *wkv, const float *q_w,
                          const float *k_w, void *h, float *gate_out, hipStream_t stream);

/* [host] ENGRAM_STATIC_SCRATCH_BYTES, the largest workspace engram_forward_static
 * can stand in for. */
size_t engram_forward_static_max_bytes(void);

/*
 * The whole layer with the block-scaled FP8 weight: engram_hash,
 * engram_gather_mx, engram_project_mx and engram_gate in one call. Arguments
 * as for engram_forward, except the weight (w_codes, w_scales as for
 * engram_project_mx); desc->row_format must be ENGRAM_ROW_E4M3_E8M0_264 and h
 * is bf16. The workspace holds row ids, the rows' codes and scales, kv and the
 * projection's workspace.
 * Errors: as engram_forward.
 */
size_t engram_forward_mx_workspace_size(const engram_hash_params *params,
                                        const engram_forward_desc *desc);
int engram_forward_mx(const engram_hash_params *params, const engram_forward_desc *desc,
                      const int32_t *ids, const int32_t *hist_in, int32_t *hist_out,
                      const void *table, const void *w_codes, const void *w_scales,
                      const float *q_w, const float *k_w, void *h, float *gate_out,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Step 5 with the short convolution branch ([P5] §4.1-§4.2), given kv.
 * Arguments as engram_gate, plus:
 *   conv      [host] the branch's shape, weights and history (engram_short_conv)
 *   workspace device, >= engram_gate_conv_workspace_size bytes, 256-byte
 *             aligned: each token's gates and mean(v^2)
 * The history is read for the chunk's first (w - 1) dilation positions and,
 * when state_v_out is set, replaced by the last L positions of history + chunk.
 * Errors: ENGRAM_EINVAL, ENGRAM_ESHAPE, ENGRAM_EWORKSPACE, ENGRAM_EHIP.
 */
size_t engram_gate_conv_workspace_size(const engram_forward_desc *desc);
int engram_gate_conv(const engram_forward_desc *desc, const engram_short_conv *conv,
                     const int32_t *ids, int32_t raw_vocab, const void *kv, const float *q_w,
                     const float *k_w, void *h, float *gate_out, void *workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * Steps 1-5 with the short convolution branch: engram_forward with
 * engram_gate_conv in place of engram_gate. Arguments as engram_forward, plus
 * conv as engram_gate_conv.
 * Errors: as engram_forward.
 */
size_t engram_forward_conv_workspace_size(const engram_hash_params *params,
                                          const engram_forward_desc *desc);
int engram_forward_conv(const engram_hash_params *params, const engram_forward_desc *desc,
                        const engram_short_conv *conv, const int32_t *ids,
                        const int32_t *hist_in, int32_t *hist_out, const void *table,
                        const void *wkv, const float *q_w, const float *k_w, void *h,
                        float *gate_out, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ENGRAM_H */

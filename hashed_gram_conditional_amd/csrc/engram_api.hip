// C ABI of the Engram layer forward: argument validation on the host, then the
// stage launches on the caller's stream. Declarations and the contract of every
// entry point are in include/engram.h.
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "common.h"

namespace {

constexpr int64_t kInt63Max = INT64_MAX;

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// batch * seq when both are >= 0 and the product is at most `limit`, else -1
// (so a product beyond int64 cannot wrap into an accepted count).
int64_t token_count(int64_t batch, int64_t seq, int64_t limit) {
  if (batch < 0 || seq < 0) return -1;
  if (seq > 0 && batch > limit / seq) return -1;
  return batch * seq;
}

// ---- deterministic Miller-Rabin for 64-bit integers --------------------------
// The bases 2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31 and 37 decide primality for
// every n < 3.3 * 10^24 (Sorenson & Webster, "Strong pseudoprimes to twelve
// prime bases", Math. Comp. 86, 2017).
uint64_t mulmod(uint64_t a, uint64_t b, uint64_t m) {
  return (uint64_t)((unsigned __int128)a * b % m);
}

uint64_t powmod(uint64_t a, uint64_t e, uint64_t m) {
  uint64_t r = 1 % m;
  a %= m;
  while (e) {
    if (e & 1) r = mulmod(r, a, m);
    a = mulmod(a, a, m);
    e >>= 1;
  }
  return r;
}

bool is_prime_mr(uint64_t n) {
  static const uint64_t bases[] = {2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37};
  if (n < 2) return false;
  for (uint64_t p : bases) {
    if (n % p == 0) return n == p;
  }
  uint64_t d = n - 1;
  int s = 0;
  while ((d & 1) == 0) {
    d >>= 1;
    ++s;
  }
  for (uint64_t a : bases) {
    uint64_t x = powmod(a, d, n);
    if (x == 1 || x == n - 1) continue;
    bool composite = true;
    for (int i = 1; i < s; ++i) {
      x = mulmod(x, x, n);
      if (x == n - 1) {
        composite = false;
        break;
      }
    }
    if (composite) return false;
  }
  return true;
}

// ---- validation -----------------------------------------------------------------
int check_hash_params(const engram_hash_params *p) {
  if (p == nullptr) return ENGRAM_EINVAL;
  if (p->raw_vocab < 1 || p->compressed_vocab < 1 || p->reserved != 0) return ENGRAM_EINVAL;
  if (p->max_ngram < 2 || p->max_ngram > ENGRAM_MAX_NGRAM || p->heads < 1) return ENGRAM_ESHAPE;
  if ((int64_t)(p->max_ngram - 1) * p->heads > ENGRAM_MAX_SEGMENTS) return ENGRAM_ESHAPE;
  if (p->pad_id < 0 || p->pad_id >= p->compressed_vocab) return ENGRAM_EINVAL;
  if (p->token_map == nullptr || !aligned(p->token_map, 4)) return ENGRAM_EINVAL;
  const int64_t bound = kInt63Max / p->compressed_vocab;
  for (int i = 0; i < p->max_ngram; ++i) {
    const int64_t m = p->multipliers[i];
    if (m < 1 || m > bound || (m & 1) == 0) return ENGRAM_EMULT;
  }
  const int S = (p->max_ngram - 1) * p->heads;
  int64_t acc = 0;
  for (int j = 0; j < S; ++j) {
    const int64_t pr = p->primes[j];
    if (pr < 2 || pr > (int64_t)UINT32_MAX) return ENGRAM_EPRIMES;
    if (p->offsets[j] != acc) return ENGRAM_EPRIMES;
    acc += pr;
  }
  return ENGRAM_OK;
}

int64_t total_rows(const engram_hash_params *p) {
  const int S = (p->max_ngram - 1) * p->heads;
  return p->offsets[S - 1] + p->primes[S - 1];
}

// Kernel arguments for `layers` validated parameter sets that agree on every
// shared field (checked by check_layer_params).
EngramHashArgs make_hash_args(const engram_hash_params *p, int layers) {
  EngramHashArgs a;
  memset(&a, 0, sizeof(a));
  a.raw_vocab = p->raw_vocab;
  a.compressed_vocab = p->compressed_vocab;
  a.max_ngram = p->max_ngram;
  a.heads = p->heads;
  a.segments = (p->max_ngram - 1) * p->heads;
  a.pad_id = p->pad_id;
  a.layers = layers;
  for (int l = 0; l < layers; ++l) {
    const engram_hash_params *q = p + l;
    for (int i = 0; i < q->max_ngram; ++i) a.mult[l][i] = (uint64_t)q->multipliers[i];
    for (int j = 0; j < a.segments; ++j) {
      const int js = l * a.segments + j;
      a.prime[js] = (uint32_t)q->primes[j];
      a.recip[js] = UINT64_MAX / (uint64_t)q->primes[j];
      a.offset[js] = q->offsets[j];
    }
  }
  return a;
}

// Several layers hashed together: each set valid on its own, all sharing the
// token map and its vocabularies, the n-gram shape and the pad id.
int check_layer_params(const engram_hash_params *p, int32_t layers) {
  if (p == nullptr) return ENGRAM_EINVAL;
  if (layers < 1 || layers > ENGRAM_MAX_LAYERS) return ENGRAM_ESHAPE;
  for (int32_t l = 0; l < layers; ++l) {
    const int rc = check_hash_params(p + l);
    if (rc != ENGRAM_OK) return rc;
    const engram_hash_params &q = p[l];
    if (q.raw_vocab != p->raw_vocab || q.compressed_vocab != p->compressed_vocab ||
        q.max_ngram != p->max_ngram || q.heads != p->heads || q.pad_id != p->pad_id ||
        q.token_map != p->token_map)
      return ENGRAM_EINVAL;
  }
  if ((int64_t)layers * (p->max_ngram - 1) * p->heads > ENGRAM_MAX_TOTAL_SEGMENTS)
    return ENGRAM_ESHAPE;
  return ENGRAM_OK;
}

int check_desc(const engram_forward_desc *d) {
  if (d == nullptr) return ENGRAM_EINVAL;
  if (token_count(d->batch, d->seq, INT32_MAX) < 0 || d->table_rows < 0) return ENGRAM_ESHAPE;
  if (d->hc < 1 || d->hc > 8) return ENGRAM_ESHAPE;
  if (d->dim < 8 || d->dim % 8 != 0 || d->dim > 8192) return ENGRAM_ESHAPE;
  if (d->row_format != ENGRAM_ROW_E4M3_E8M0_264 && d->row_format != ENGRAM_ROW_F32)
    return ENGRAM_EINVAL;
  if (d->row_format == ENGRAM_ROW_E4M3_E8M0_264 && d->row_dim != ENGRAM_ROW_DIM_E4M3)
    return ENGRAM_ESHAPE;
  if (d->row_format == ENGRAM_ROW_F32 && (d->row_dim < 4 || d->row_dim % 4 != 0))
    return ENGRAM_ESHAPE;
  if (!(d->eps >= 0.f) || !(d->gate_clamp >= 0.f)) return ENGRAM_EINVAL;
  if (d->gate_mode != ENGRAM_GATE_SIGNED_SQRT && d->gate_mode != ENGRAM_GATE_PLAIN)
    return ENGRAM_EINVAL;
  if (d->wkv_ld < 0) return ENGRAM_ESHAPE;
  return ENGRAM_OK;
}

int check_conv(const engram_short_conv *c) {
  if (c == nullptr || c->reserved != 0) return ENGRAM_EINVAL;
  if (c->taps < 1 || c->taps > ENGRAM_MAX_CONV_TAPS || c->dilation < 1) return ENGRAM_ESHAPE;
  if ((int64_t)(c->taps - 1) * c->dilation > ENGRAM_MAX_CONV_HISTORY) return ENGRAM_ESHAPE;
  if (!(c->eps > 0.f) || !(c->eps < INFINITY)) return ENGRAM_EINVAL;
  if (c->weight == nullptr || !aligned(c->weight, 16) || !aligned(c->norm_weight, 16))
    return ENGRAM_EINVAL;
  if ((c->state_v_in == nullptr) != (c->state_s_in == nullptr) ||
      (c->state_v_out == nullptr) != (c->state_s_out == nullptr))
    return ENGRAM_EINVAL;
  if (!aligned(c->state_v_in, 16) || !aligned(c->state_v_out, 16) ||
      !aligned(c->state_s_in, 4) || !aligned(c->state_s_out, 4))
    return ENGRAM_EINVAL;
  return ENGRAM_OK;
}

EngramConvArgs make_conv_args(const engram_short_conv *c) {
  EngramConvArgs a;
  a.taps = c->taps;
  a.dilation = c->dilation;
  a.history = (c->taps - 1) * c->dilation;
  a.eps = c->eps;
  a.weight = c->weight;
  a.norm_weight = c->norm_weight;
  a.state_v_in = c->state_v_in;
  a.state_s_in = c->state_s_in;
  a.state_v_out = c->state_v_out;
  a.state_s_out = c->state_s_out;
  return a;
}

// The bf16 projection kernels address each 256-row operand panel through a
// buffer resource whose byte count (rows * K * 2) and byte offsets are 32-bit,
// and index their grids with int tile products: K up to 2^20 keeps a panel below
// 2^30 bytes, and the largest grid (128-wide tiles of 512 threads) must stay
// within 2^32 threads.
constexpr int64_t kMaxProjectInDim = (int64_t)1 << 20;

bool bf16_projection_shape_ok(int64_t tokens, int64_t in_dim, int64_t out_dim) {
  if (in_dim > kMaxProjectInDim) return false;
  const int64_t tiles_m = (tokens + 255) / 256;
  const int64_t tiles_n = (out_dim + 127) / 128;
  return tiles_m * tiles_n <= ((int64_t)1 << 32) / 512 - 1;
}

// Row stride of wkv in elements: 0 means in_dim (dense rows). Otherwise at least
// in_dim and a multiple of 16 bytes, so that every row starts 16-byte aligned;
// for bf16 within the same 32-bit panel bound as in_dim.
int wkv_row_stride(int64_t ld, int64_t in_dim, bool f32, int64_t *out) {
  if (ld == 0) ld = in_dim;
  if (ld < in_dim || ld % (f32 ? 4 : 8) != 0) return ENGRAM_ESHAPE;
  if (!f32 && ld > kMaxProjectInDim) return ENGRAM_ESHAPE;
  *out = ld;
  return ENGRAM_OK;
}

// The stage entry points (engram_gate, engram_gate_conv) know only the raw ids;
// the fused ones apply the hash's full rule, so a token map value outside
// [0, V') makes the position DEAD in the gate exactly as in its row ids.
EngramDeadRule raw_id_rule(int32_t raw_vocab) { return EngramDeadRule{raw_vocab, 0, nullptr}; }

EngramDeadRule hash_rule(const engram_hash_params *p) {
  return EngramDeadRule{p->raw_vocab, p->compressed_vocab, p->token_map};
}

// engram_forward folds the gate's two scale arrays into one (the same fp32
// products, so the same bits) when the call has at least this many tokens: the
// gate then reads half the scale bytes per token (12 % faster at 32768 tokens,
// 8 % at 2048 with the fold's launch counted), while at 1024 tokens and below the
// extra launch costs more than it saves.
constexpr int64_t kFoldMinTokens = 2048;

// engram_forward forms and gathers the rows in one launch (one block per token)
// for calls of at most this many tokens; larger calls hash with several tokens
// per block and gather with the whole grid.
constexpr int64_t kHashGatherMaxTokens = 2048;

size_t folded_scales_bytes(const engram_forward_desc *d) {
  return align256((size_t)d->hc * (size_t)d->dim * sizeof(float));
}

// Bytes of engram_forward's workspace before the projection's own part: row
// ids, e, kv and the folded gate scales.
size_t forward_base_bytes(const engram_hash_params *params, const engram_forward_desc *desc) {
  const int64_t ntok = desc->batch * desc->seq;
  const int64_t S = (int64_t)(params->max_ngram - 1) * params->heads;
  const size_t esz = desc->row_format == ENGRAM_ROW_F32 ? 4 : 2;
  const int64_t in_dim = S * desc->row_dim;
  const int64_t out_dim = (int64_t)(desc->hc + 1) * desc->dim;
  return align256((size_t)ntok * S * 8) + align256((size_t)ntok * in_dim * esz) +
         align256((size_t)ntok * out_dim * esz) + folded_scales_bytes(desc);
}

size_t gate_conv_workspace(const engram_forward_desc *d) {
  return align256((size_t)(d->batch * d->seq) * (size_t)(d->hc + 1) * sizeof(float));
}

// The address through which the kernels read a table: device (or managed)
// memory as it is, pinned host memory through its mapping into the device's
// address space, so the kernels then read the rows over the host link. Memory
// the device cannot reach (pageable host memory, an unknown pointer) would
// fault in a kernel and is rejected here instead.
int resolve_table(const void *table, int64_t table_rows, const void **dev, bool *host) {
  *dev = table;
  *host = false;
  if (table_rows == 0) return ENGRAM_OK;
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, table) != hipSuccess) {
    (void)hipGetLastError();
    return ENGRAM_EINVAL;
  }
  if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) return ENGRAM_OK;
  if (a.type == hipMemoryTypeHost && a.devicePointer != nullptr) {
    *dev = a.devicePointer;
    *host = true;
    return ENGRAM_OK;
  }
  return ENGRAM_EINVAL;
}

// The last HIP error an entry point returned ENGRAM_EHIP for, per host thread.
thread_local hipError_t g_last_hip_error = hipSuccess;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return ENGRAM_OK;
  g_last_hip_error = e;
  return ENGRAM_EHIP;
}

}  // namespace

extern "C" {

const char *engram_status_string(int status) {
  switch (status) {
    case ENGRAM_OK: return "ok";
    case ENGRAM_EINVAL: return "invalid argument (null or misaligned pointer, bad value)";
    case ENGRAM_EVOCAB: return "compressed vocabulary does not match the token map";
    case ENGRAM_EMULT: return "multiplier even, < 1 or above (2^63-1)/compressed_vocab";
    case ENGRAM_ESHAPE: return "inconsistent shapes";
    case ENGRAM_EWORKSPACE: return "workspace missing or too small";
    case ENGRAM_EHIP: return "HIP launch failed";
    case ENGRAM_EPRIMES: return "bad primes/offsets or rows beyond the table";
    case ENGRAM_ESCRATCH:
      return "the call needs more scratch than engram_forward_static's static array holds";
    default: return "unknown status";
  }
}

const char *engram_last_hip_error(void) { return hipGetErrorString(g_last_hip_error); }

size_t engram_sizeof_hash_params(void) { return sizeof(engram_hash_params); }

size_t engram_sizeof_forward_desc(void) { return sizeof(engram_forward_desc); }

size_t engram_sizeof_short_conv(void) { return sizeof(engram_short_conv); }

int engram_make_primes(int64_t base, int32_t count, int64_t *primes_out, int64_t *offsets_out,
                       int64_t *total_rows_out) {
  if (count < 0 || base < 2 || (count > 0 && (primes_out == nullptr || offsets_out == nullptr)))
    return ENGRAM_EINVAL;
  uint64_t n = (uint64_t)base;
  int64_t acc = 0;
  for (int32_t j = 0; j < count; ++n) {
    if (n > UINT32_MAX) return ENGRAM_EINVAL;
    if (is_prime_mr(n)) {
      primes_out[j] = (int64_t)n;
      offsets_out[j] = acc;
      acc += (int64_t)n;
      ++j;
    }
  }
  if (total_rows_out) *total_rows_out = acc;
  return ENGRAM_OK;
}

int engram_make_layer_primes(int64_t base, int32_t layers, int32_t per_layer,
                             int64_t *primes_out, int64_t *offsets_out, int64_t *rows_out) {
  if (layers < 1 || per_layer < 0) return ENGRAM_EINVAL;
  const int64_t count = (int64_t)layers * per_layer;
  if (count > INT32_MAX) return ENGRAM_EINVAL;
  // One ascending sequence, dealt to the layers in order; offsets restart per layer.
  int rc = engram_make_primes(base, (int32_t)count, primes_out, offsets_out, nullptr);
  if (rc != ENGRAM_OK) return rc;
  for (int32_t l = 0; l < layers; ++l) {
    int64_t acc = 0;
    for (int32_t j = 0; j < per_layer; ++j) {
      const int64_t k = (int64_t)l * per_layer + j;
      offsets_out[k] = acc;
      acc += primes_out[k];
    }
    if (rows_out) rows_out[l] = acc;
  }
  return ENGRAM_OK;
}

int engram_check_token_map(const int32_t *token_map, int32_t raw_vocab,
                           int32_t compressed_vocab) {
  if (token_map == nullptr || raw_vocab < 1 || compressed_vocab < 1) return ENGRAM_EINVAL;
  uint8_t *seen = (uint8_t *)calloc((size_t)compressed_vocab, 1);
  if (seen == nullptr) return ENGRAM_EINVAL;
  int32_t hit = 0;
  int rc = ENGRAM_OK;
  for (int32_t i = 0; i < raw_vocab; ++i) {
    const int32_t v = token_map[i];
    if (v < 0 || v >= compressed_vocab) {
      rc = ENGRAM_EVOCAB;
      break;
    }
    if (!seen[v]) {
      seen[v] = 1;
      ++hit;
    }
  }
  if (rc == ENGRAM_OK && hit != compressed_vocab) rc = ENGRAM_EVOCAB;
  free(seen);
  return rc;
}

int engram_hash_layers(const engram_hash_params *params, int32_t layers, const int32_t *ids,
                       int64_t batch, int64_t seq, const int32_t *hist_in, int32_t *hist_out,
                       int64_t *row_ids, hipStream_t stream) {
  int rc = check_layer_params(params, layers);
  if (rc != ENGRAM_OK) return rc;
  const int64_t ntok = token_count(batch, seq, (int64_t)INT32_MAX * 64);
  if (ntok < 0) return ENGRAM_ESHAPE;
  if (ntok > 0 && (ids == nullptr || row_ids == nullptr)) return ENGRAM_EINVAL;
  if (!aligned(ids, 4) || !aligned(row_ids, 8) || !aligned(hist_in, 4) || !aligned(hist_out, 4))
    return ENGRAM_EINVAL;
  const EngramHashArgs a = make_hash_args(params, layers);
  return hip_status(engram_launch_hash(a, params->token_map, ids, batch, seq, hist_in, hist_out,
                                       row_ids, stream));
}

int engram_hash(const engram_hash_params *params, const int32_t *ids, int64_t batch,
                int64_t seq, const int32_t *hist_in, int32_t *hist_out, int64_t *row_ids,
                hipStream_t stream) {
  return engram_hash_layers(params, 1, ids, batch, seq, hist_in, hist_out, row_ids, stream);
}

int engram_gather(const void *table, int64_t table_rows, int32_t row_format, int32_t row_dim,
                  const int64_t *row_ids, int64_t n_ids, void *out, hipStream_t stream) {
  if (n_ids < 0 || table_rows < 0) return ENGRAM_ESHAPE;
  if (row_format == ENGRAM_ROW_E4M3_E8M0_264) {
    if (row_dim != ENGRAM_ROW_DIM_E4M3) return ENGRAM_ESHAPE;
  } else if (row_format == ENGRAM_ROW_F32) {
    if (row_dim < 4 || row_dim % 4 != 0) return ENGRAM_ESHAPE;
  } else {
    return ENGRAM_EINVAL;
  }
  if (n_ids == 0) return ENGRAM_OK;
  if (row_ids == nullptr || out == nullptr || (table == nullptr && table_rows > 0))
    return ENGRAM_EINVAL;
  if (!aligned(table, 16) || !aligned(row_ids, 8) || !aligned(out, 16)) return ENGRAM_EINVAL;
  bool host = false;
  const int rc = resolve_table(table, table_rows, &table, &host);
  if (rc != ENGRAM_OK) return rc;
  hipError_t e;
  if (row_format == ENGRAM_ROW_E4M3_E8M0_264)
    e = engram_launch_gather_e4m3((const uint8_t *)table, table_rows, row_ids, n_ids,
                                  (uint16_t *)out, host, stream);
  else
    e = engram_launch_gather_f32((const float *)table, table_rows, row_dim, row_ids, n_ids,
                                 (float *)out, stream);
  return hip_status(e);
}

int engram_gather_rows(const void *table, int64_t table_rows, const int64_t *row_ids,
                       int64_t n_ids, void *out, hipStream_t stream) {
  if (n_ids < 0 || table_rows < 0) return ENGRAM_ESHAPE;
  if (n_ids == 0) return ENGRAM_OK;
  if (row_ids == nullptr || out == nullptr || (table == nullptr && table_rows > 0))
    return ENGRAM_EINVAL;
  if (!aligned(table, 8) || !aligned(row_ids, 8) || !aligned(out, 8)) return ENGRAM_EINVAL;
  bool host = false;
  const int rc = resolve_table(table, table_rows, &table, &host);
  if (rc != ENGRAM_OK) return rc;
  return hip_status(engram_launch_gather_rows((const uint8_t *)table, table_rows, row_ids,
                                              n_ids, (uint8_t *)out, host, stream));
}

int engram_gather_mx(const void *table, int64_t table_rows, const int64_t *row_ids,
                     int64_t n_ids, void *codes, void *scales, hipStream_t stream) {
  if (n_ids < 0 || table_rows < 0) return ENGRAM_ESHAPE;
  if (n_ids == 0) return ENGRAM_OK;
  if (row_ids == nullptr || codes == nullptr || scales == nullptr ||
      (table == nullptr && table_rows > 0))
    return ENGRAM_EINVAL;
  if (!aligned(table, 8) || !aligned(row_ids, 8) || !aligned(codes, 16) || !aligned(scales, 8))
    return ENGRAM_EINVAL;
  bool host = false;
  const int rc = resolve_table(table, table_rows, &table, &host);
  if (rc != ENGRAM_OK) return rc;
  return hip_status(engram_launch_gather_mx((const uint8_t *)table, table_rows, row_ids, n_ids,
                                            (uint8_t *)codes, (uint8_t *)scales, host, stream));
}

size_t engram_project_mx_workspace_size(int64_t tokens, int32_t segments, int64_t out_dim) {
  if (tokens <= 0 || segments < 1 || out_dim < 1) return 0;
  size_t bytes = 0;
  if (engram_gemm_mx_workspace(tokens, out_dim, segments, &bytes) != hipSuccess) return 0;
  return bytes;
}

int engram_project_mx(const void *e_codes, const void *e_scales, int32_t segments,
                      const void *w_codes, const void *w_scales, void *kv, int64_t tokens,
                      int64_t out_dim, void *workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  if (tokens < 0 || segments < 1 || segments > ENGRAM_MAX_SEGMENTS || out_dim < 1)
    return ENGRAM_ESHAPE;
  if (out_dim % 8 || tokens > INT32_MAX || out_dim > INT32_MAX) return ENGRAM_ESHAPE;
  if (!bf16_projection_shape_ok(tokens, (int64_t)segments * ENGRAM_ROW_DIM_E4M3, out_dim))
    return ENGRAM_ESHAPE;
  if (tokens == 0) return ENGRAM_OK;
  if (e_codes == nullptr || e_scales == nullptr || w_codes == nullptr || w_scales == nullptr ||
      kv == nullptr)
    return ENGRAM_EINVAL;
  if (!aligned(e_codes, 16) || !aligned(e_scales, 4) || !aligned(w_codes, 16) ||
      !aligned(w_scales, 4) || !aligned(kv, 16))
    return ENGRAM_EINVAL;
  if (workspace != nullptr) {
    if (!aligned(workspace, 256) ||
        workspace_bytes < engram_project_mx_workspace_size(tokens, segments, out_dim))
      return ENGRAM_EWORKSPACE;
  }
  return hip_status(engram_launch_gemm_mx((const uint8_t *)w_codes, (const uint8_t *)w_scales,
                                          (const uint8_t *)e_codes, (const uint8_t *)e_scales,
                                          segments, (uint16_t *)kv, tokens, out_dim, workspace,
                                          workspace_bytes, stream));
}

size_t engram_project_workspace_size(int64_t tokens, int64_t in_dim, int64_t out_dim,
                                     int32_t act_f32) {
  if (act_f32 != 0 || tokens <= 0 || in_dim < 1 || out_dim < 1) return 0;
  size_t bytes = 0;
  if (engram_gemm_bf16_workspace(tokens, out_dim, in_dim, &bytes) != hipSuccess) return 0;
  return bytes;
}

int engram_project(const void *e, const void *wkv, void *kv, int64_t tokens, int64_t in_dim,
                   int64_t out_dim, int64_t wkv_ld, int32_t act_f32, void *workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  if (tokens < 0 || in_dim < 1 || out_dim < 1) return ENGRAM_ESHAPE;
  if (act_f32 != 0 && act_f32 != 1) return ENGRAM_EINVAL;
  if (act_f32) {
    if (in_dim % 4 || out_dim % 4) return ENGRAM_ESHAPE;
  } else {
    if (in_dim % 64 || out_dim % 8) return ENGRAM_ESHAPE;
  }
  if (tokens > INT32_MAX || out_dim > INT32_MAX || in_dim > INT32_MAX) return ENGRAM_ESHAPE;
  if (!act_f32 && !bf16_projection_shape_ok(tokens, in_dim, out_dim)) return ENGRAM_ESHAPE;
  int64_t ldw = 0;
  const int rc = wkv_row_stride(wkv_ld, in_dim, act_f32 != 0, &ldw);
  if (rc != ENGRAM_OK) return rc;
  if (tokens == 0) return ENGRAM_OK;
  if (e == nullptr || wkv == nullptr || kv == nullptr) return ENGRAM_EINVAL;
  if (!aligned(e, 16) || !aligned(wkv, 16) || !aligned(kv, 16)) return ENGRAM_EINVAL;
  if (workspace != nullptr) {
    if (!aligned(workspace, 256) ||
        workspace_bytes < engram_project_workspace_size(tokens, in_dim, out_dim, act_f32))
      return ENGRAM_EWORKSPACE;
  }
  hipError_t err =
      act_f32 ? engram_launch_gemm_f32((const float *)e, (const float *)wkv, ldw, (float *)kv,
                                       tokens, out_dim, in_dim, stream)
              : engram_launch_gemm_bf16((const uint16_t *)e, (const uint16_t *)wkv, ldw,
                                        (uint16_t *)kv, tokens, out_dim, in_dim, workspace,
                                        workspace_bytes, stream);
  return hip_status(err);
}

int engram_gate(const engram_forward_desc *desc, const int32_t *ids, int32_t raw_vocab,
                const void *kv, const float *q_w, const float *k_w, void *h, float *gate_out,
                hipStream_t stream) {
  int rc = check_desc(desc);
  if (rc != ENGRAM_OK) return rc;
  if (raw_vocab < 1) return ENGRAM_EINVAL;
  const int64_t ntok = desc->batch * desc->seq;
  if (ntok == 0) return ENGRAM_OK;
  if (ids == nullptr || kv == nullptr || q_w == nullptr || k_w == nullptr || h == nullptr)
    return ENGRAM_EINVAL;
  if (!aligned(ids, 4) || !aligned(kv, 16) || !aligned(q_w, 16) || !aligned(k_w, 16) ||
      !aligned(h, 16) || !aligned(gate_out, 4))
    return ENGRAM_EINVAL;
  if (ntok > INT32_MAX) return ENGRAM_ESHAPE;
  return hip_status(engram_launch_gate(desc->row_format == ENGRAM_ROW_F32, ids,
                                       raw_id_rule(raw_vocab), kv, q_w, k_w, h, gate_out,
                                       nullptr, ntok, desc->hc,
                                       desc->dim, desc->eps, desc->gate_clamp, desc->gate_mode,
                                       stream));
}

int engram_fold_gate_weights(const float *q_w, const float *k_w, int32_t hc, int32_t dim,
                             float *qk_w, hipStream_t stream) {
  if (hc < 1 || hc > 8 || dim < 8 || dim % 8 != 0 || dim > 8192) return ENGRAM_ESHAPE;
  if (q_w == nullptr || k_w == nullptr || qk_w == nullptr) return ENGRAM_EINVAL;
  if (!aligned(q_w, 16) || !aligned(k_w, 16) || !aligned(qk_w, 16)) return ENGRAM_EINVAL;
  return hip_status(engram_launch_fold_gate_weights(q_w, k_w, qk_w, hc, dim, stream));
}

int engram_gate_folded(const engram_forward_desc *desc, const int32_t *ids, int32_t raw_vocab,
                       const void *kv, const float *qk_w, void *h, float *gate_out,
                       hipStream_t stream) {
  int rc = check_desc(desc);
  if (rc != ENGRAM_OK) return rc;
  if (raw_vocab < 1) return ENGRAM_EINVAL;
  const int64_t ntok = desc->batch * desc->seq;
  if (ntok == 0) return ENGRAM_OK;
  if (ids == nullptr || kv == nullptr || qk_w == nullptr || h == nullptr) return ENGRAM_EINVAL;
  if (!aligned(ids, 4) || !aligned(kv, 16) || !aligned(qk_w, 16) || !aligned(h, 16) ||
      !aligned(gate_out, 4))
    return ENGRAM_EINVAL;
  return hip_status(engram_launch_gate(desc->row_format == ENGRAM_ROW_F32, ids,
                                       raw_id_rule(raw_vocab), kv, qk_w, nullptr, h, gate_out,
                                       nullptr, ntok, desc->hc,
                                       desc->dim, desc->eps, desc->gate_clamp, desc->gate_mode,
                                       stream));
}

int engram_project_gate_sums(const engram_forward_desc *desc, const void *e, int64_t in_dim,
                             const void *wkv, const void *h, const float *qk_w, void *kv,
                             hipStream_t stream) {
  int rc = check_desc(desc);
  if (rc != ENGRAM_OK) return rc;
  if (desc->row_format != ENGRAM_ROW_E4M3_E8M0_264) return ENGRAM_EINVAL;
  if (desc->dim % 256 != 0 || in_dim < 1 || in_dim % 64 != 0) return ENGRAM_ESHAPE;
  const int64_t ntok = desc->batch * desc->seq;
  const int64_t out_dim = (int64_t)(desc->hc + 1) * desc->dim;
  if (ntok > INT32_MAX || in_dim > INT32_MAX) return ENGRAM_ESHAPE;
  if (!bf16_projection_shape_ok(ntok, in_dim, out_dim)) return ENGRAM_ESHAPE;
  int64_t ldw = 0;
  if ((rc = wkv_row_stride(desc->wkv_ld, in_dim, false, &ldw)) != ENGRAM_OK) return rc;
  if (ntok == 0) return ENGRAM_OK;
  if (e == nullptr || wkv == nullptr || h == nullptr || qk_w == nullptr || kv == nullptr)
    return ENGRAM_EINVAL;
  if (!aligned(e, 16) || !aligned(wkv, 16) || !aligned(h, 16) || !aligned(qk_w, 16) ||
      !aligned(kv, 16))
    return ENGRAM_EINVAL;
  return hip_status(engram_launch_gemm_bf16_sums((const uint16_t *)e, (const uint16_t *)wkv, ldw,
                                                 (const uint16_t *)h, qk_w, (uint16_t *)kv, ntok,
                                                 desc->hc, desc->dim, in_dim, stream));
}

int engram_project_mx_gate_sums(const engram_forward_desc *desc, const void *e_codes,
                                const void *e_scales, int32_t segments, const void *w_codes,
                                const void *w_scales, const void *h, const float *qk_w,
                                void *kv, hipStream_t stream) {
  const int rc = check_desc(desc);
  if (rc != ENGRAM_OK) return rc;
  if (desc->row_format != ENGRAM_ROW_E4M3_E8M0_264) return ENGRAM_EINVAL;
  if (segments < 1 || segments > ENGRAM_MAX_SEGMENTS || desc->dim % 256 != 0)
    return ENGRAM_ESHAPE;
  const int64_t ntok = desc->batch * desc->seq;
  const int64_t out_dim = (int64_t)(desc->hc + 1) * desc->dim;
  if (ntok > INT32_MAX) return ENGRAM_ESHAPE;
  if (!bf16_projection_shape_ok(ntok, (int64_t)segments * ENGRAM_ROW_DIM_E4M3, out_dim))
    return ENGRAM_ESHAPE;
  if (ntok == 0) return ENGRAM_OK;
  if (e_codes == nullptr || e_scales == nullptr || w_codes == nullptr || w_scales == nullptr ||
      h == nullptr || qk_w == nullptr || kv == nullptr)
    return ENGRAM_EINVAL;
  if (!aligned(e_codes, 16) || !aligned(e_scales, 4) || !aligned(w_codes, 16) ||
      !aligned(w_scales, 4) || !aligned(h, 16) || !aligned(qk_w, 16) || !aligned(kv, 16))
    return ENGRAM_EINVAL;
  return hip_status(engram_launch_gemm_mx_sums(
      (const uint8_t *)w_codes, (const uint8_t *)w_scales, (const uint8_t *)e_codes,
      (const uint8_t *)e_scales, segments, (const uint16_t *)h, qk_w, (uint16_t *)kv, ntok,
      desc->hc, desc->dim, stream));
}

int engram_gate_sums(const engram_forward_desc *desc, const int32_t *ids, int32_t raw_vocab,
                     const void *kv, void *h, float *gate_out, hipStream_t stream) {
  const int rc = check_desc(desc);
  if (rc != ENGRAM_OK) return rc;
  if (raw_vocab < 1 || desc->row_format != ENGRAM_ROW_E4M3_E8M0_264) return ENGRAM_EINVAL;
  if (desc->dim % 256 != 0) return ENGRAM_ESHAPE;
  const int64_t ntok = desc->batch * desc->seq;
  if (ntok == 0) return ENGRAM_OK;
  if (ids == nullptr || kv == nullptr || h == nullptr) return ENGRAM_EINVAL;
  if (!aligned(ids, 4) || !aligned(kv, 16) || !aligned(h, 16) || !aligned(gate_out, 4))
    return ENGRAM_EINVAL;
  if (ntok > INT32_MAX) return ENGRAM_ESHAPE;
  return hip_status(engram_launch_gate_sums(ids, raw_id_rule(raw_vocab), kv, h, gate_out, nullptr,
                                            ntok, desc->hc, desc->dim, desc->eps,
                                            desc->gate_clamp, desc->gate_mode, stream));
}

int engram_gate_conv_sums(const engram_forward_desc *desc, const engram_short_conv *conv,
                          const int32_t *ids, int32_t raw_vocab, const void *kv, void *h,
                          float *gate_out, void *workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  int rc = check_desc(desc);
  if (rc != ENGRAM_OK) return rc;
  rc = check_conv(conv);
  if (rc != ENGRAM_OK) return rc;
  if (raw_vocab < 1 || desc->row_format != ENGRAM_ROW_E4M3_E8M0_264) return ENGRAM_EINVAL;
  if (desc->dim % 256 != 0) return ENGRAM_ESHAPE;
  const int64_t ntok = desc->batch * desc->seq;
  if (ntok > INT32_MAX) return ENGRAM_ESHAPE;
  if (ntok > 0) {
    if (ids == nullptr || kv == nullptr || h == nullptr) return ENGRAM_EINVAL;
    if (!aligned(ids, 4) || !aligned(kv, 16) || !aligned(h, 16) || !aligned(gate_out, 4))
      return ENGRAM_EINVAL;
    if (workspace == nullptr || workspace_bytes < gate_conv_workspace(desc) ||
        !aligned(workspace, 256))
      return ENGRAM_EWORKSPACE;
  }
  float *stats = (float *)workspace;
  if (ntok > 0) {
    const hipError_t err = engram_launch_gate_sums(ids, raw_id_rule(raw_vocab), kv, h, gate_out,
                                                   stats, ntok, desc->hc, desc->dim, desc->eps,
                                                   desc->gate_clamp, desc->gate_mode, stream);
    if (err != hipSuccess) return hip_status(err);
  }
  return hip_status(engram_launch_short_conv(false, make_conv_args(conv), ids,
                                             raw_id_rule(raw_vocab), kv, stats, h, desc->batch,
                                             desc->seq, desc->hc, desc->dim, stream));
}

int engram_transpose(const void *src, void *dst, int64_t rows, int64_t cols, int64_t dst_ld,
                     int32_t elem_bytes, hipStream_t stream) {
  if (elem_bytes != 2 && elem_bytes != 4) return ENGRAM_EINVAL;
  if (rows < 0 || cols < 0 || dst_ld < 0) return ENGRAM_ESHAPE;
  if (dst_ld == 0) dst_ld = rows;
  if (dst_ld < rows) return ENGRAM_ESHAPE;
  if (rows == 0 || cols == 0) return ENGRAM_OK;
  // the destination's extent, (cols - 1) dst_ld + rows elements, in bytes below 2^62
  if (cols > 1 && dst_ld > (((int64_t)1 << 62) / elem_bytes - rows) / (cols - 1))
    return ENGRAM_ESHAPE;
  // 64 x 64 tiles of 256 threads: at most 2^24 tiles keeps the grid within 2^32
  // threads.
  const int64_t tr = (rows + 63) / 64, tc = (cols + 63) / 64;
  if (tr > ((int64_t)1 << 24) / tc) return ENGRAM_ESHAPE;
  if (src == nullptr || dst == nullptr) return ENGRAM_EINVAL;
  if (!aligned(src, elem_bytes) || !aligned(dst, elem_bytes)) return ENGRAM_EINVAL;
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  const uintptr_t ns = (uintptr_t)(rows * cols * elem_bytes);
  const uintptr_t nd = (uintptr_t)(((cols - 1) * dst_ld + rows) * elem_bytes);
  if (s0 < d0 + nd && d0 < s0 + ns) return ENGRAM_EINVAL;      // overlapping buffers
  return hip_status(engram_launch_transpose(src, dst, rows, cols, dst_ld, elem_bytes, stream));
}

int64_t engram_wkv_row_stride(int64_t in_dim, int32_t elem_bytes) {
  if (in_dim < 1 || in_dim > kMaxProjectInDim || (elem_bytes != 2 && elem_bytes != 4)) return 0;
  int64_t bytes = (in_dim * elem_bytes + 127) / 128 * 128;
  if (bytes % 4096 == 0) bytes += 128;
  return bytes / elem_bytes;
}

size_t engram_gate_conv_workspace_size(const engram_forward_desc *desc) {
  if (check_desc(desc) != ENGRAM_OK) return 0;
  return gate_conv_workspace(desc);
}

int engram_gate_conv(const engram_forward_desc *desc, const engram_short_conv *conv,
                     const int32_t *ids, int32_t raw_vocab, const void *kv, const float *q_w,
                     const float *k_w, void *h, float *gate_out, void *workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  int rc = check_desc(desc);
  if (rc != ENGRAM_OK) return rc;
  rc = check_conv(conv);
  if (rc != ENGRAM_OK) return rc;
  if (raw_vocab < 1) return ENGRAM_EINVAL;
  const int64_t ntok = desc->batch * desc->seq;
  if (ntok > INT32_MAX) return ENGRAM_ESHAPE;
  if (ntok > 0) {
    if (ids == nullptr || kv == nullptr || q_w == nullptr || k_w == nullptr || h == nullptr)
      return ENGRAM_EINVAL;
    if (!aligned(ids, 4) || !aligned(kv, 16) || !aligned(q_w, 16) || !aligned(k_w, 16) ||
        !aligned(h, 16) || !aligned(gate_out, 4))
      return ENGRAM_EINVAL;
    if (workspace == nullptr || workspace_bytes < gate_conv_workspace(desc) ||
        !aligned(workspace, 256))
      return ENGRAM_EWORKSPACE;
  }
  const bool f32 = desc->row_format == ENGRAM_ROW_F32;
  float *stats = (float *)workspace;
  if (ntok > 0) {
    hipError_t err = engram_launch_gate(f32, ids, raw_id_rule(raw_vocab), kv, q_w, k_w, h,
                                        gate_out, stats,
                                        ntok, desc->hc, desc->dim, desc->eps, desc->gate_clamp,
                                        desc->gate_mode, stream);
    if (err != hipSuccess) return hip_status(err);
  }
  return hip_status(engram_launch_short_conv(f32, make_conv_args(conv), ids,
                                             raw_id_rule(raw_vocab), kv, stats,
                                             h, desc->batch, desc->seq, desc->hc, desc->dim,
                                             stream));
}

size_t engram_forward_workspace_size(const engram_hash_params *params,
                                     const engram_forward_desc *desc) {
  if (check_hash_params(params) != ENGRAM_OK || check_desc(desc) != ENGRAM_OK) return 0;
  const int64_t ntok = desc->batch * desc->seq;
  const int64_t S = (int64_t)(params->max_ngram - 1) * params->heads;
  const bool f32 = desc->row_format == ENGRAM_ROW_F32;
  const size_t esz = f32 ? 4 : 2;
  const int64_t in_dim = S * desc->row_dim;
  const int64_t out_dim = (int64_t)(desc->hc + 1) * desc->dim;
  return forward_base_bytes(params, desc) +
         engram_project_workspace_size(ntok, in_dim, out_dim, f32 ? 1 : 0);
}

}  // extern "C"

namespace {

// engram_forward and engram_forward_conv: steps 1-4, then the gate alone
// (conv == NULL) or the gate and the short convolution branch. With
// `gemm_ws_optional` the workspace need only hold forward_base_bytes; the
// projection then splits K over the CUs only if its partial tiles fit in the
// rest (otherwise it runs 128-wide tiles, the wide kernel's bits).
int forward_impl(const engram_hash_params *params, const engram_forward_desc *desc,
                 const engram_short_conv *conv, const int32_t *ids, const int32_t *hist_in,
                 int32_t *hist_out, const void *table, const void *wkv, const float *q_w,
                 const float *k_w, void *h, float *gate_out, void *workspace,
                 size_t workspace_bytes, hipStream_t stream, bool gemm_ws_optional = false) {
  int rc = check_hash_params(params);
  if (rc != ENGRAM_OK) return rc;
  rc = check_desc(desc);
  if (rc != ENGRAM_OK) return rc;
  if (conv != nullptr && (rc = check_conv(conv)) != ENGRAM_OK) return rc;
  if (total_rows(params) > desc->table_rows) return ENGRAM_EPRIMES;
  const int64_t ntok = desc->batch * desc->seq;
  const int64_t S = (int64_t)(params->max_ngram - 1) * params->heads;
  const bool f32 = desc->row_format == ENGRAM_ROW_F32;
  const int64_t in_dim = S * desc->row_dim;
  const int64_t out_dim = (int64_t)(desc->hc + 1) * desc->dim;
  if (!f32 && in_dim % 64) return ENGRAM_ESHAPE;
  if (ntok > INT32_MAX) return ENGRAM_ESHAPE;
  if (!f32 && !bf16_projection_shape_ok(ntok, in_dim, out_dim)) return ENGRAM_ESHAPE;
  int64_t ldw = 0;
  if ((rc = wkv_row_stride(desc->wkv_ld, in_dim, f32, &ldw)) != ENGRAM_OK) return rc;
  bool host = false;
  if (ntok > 0) {
    if (ids == nullptr || table == nullptr || wkv == nullptr || q_w == nullptr ||
        k_w == nullptr || h == nullptr)
      return ENGRAM_EINVAL;
    if (!aligned(ids, 4) || !aligned(table, 16) || !aligned(wkv, 16) || !aligned(q_w, 16) ||
        !aligned(k_w, 16) || !aligned(h, 16) || !aligned(gate_out, 4))
      return ENGRAM_EINVAL;
    const size_t need = (gemm_ws_optional ? forward_base_bytes(params, desc)
                                          : engram_forward_workspace_size(params, desc)) +
                        (conv != nullptr ? gate_conv_workspace(desc) : 0);
    if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256))
      return ENGRAM_EWORKSPACE;
    if ((rc = resolve_table(table, desc->table_rows, &table, &host)) != ENGRAM_OK) return rc;
  }
  if (!aligned(hist_in, 4) || !aligned(hist_out, 4)) return ENGRAM_EINVAL;

  // The convolution's per-token stats lead the workspace; the rest is
  // engram_forward's layout.
  float *stats = (float *)workspace;
  char *ws = (char *)workspace;
  if (conv != nullptr && ntok > 0) {
    ws += gate_conv_workspace(desc);
    workspace_bytes -= gate_conv_workspace(desc);
  }
  const size_t esz = f32 ? 4 : 2;
  int64_t *row_ids = (int64_t *)ws;
  void *e = ws + align256((size_t)ntok * S * 8);
  void *kv = (char *)e + align256((size_t)ntok * in_dim * esz);
  float *qk_w = (float *)((char *)kv + align256((size_t)ntok * out_dim * esz));
  char *gemm_ws = (char *)qk_w + folded_scales_bytes(desc);
  const size_t gemm_ws_bytes = workspace_bytes - (size_t)(gemm_ws - ws);

  const EngramHashArgs a = make_hash_args(params, 1);
  hipError_t err = hipSuccess;
  // Decode-sized calls on an HBM table form and gather each token's rows in one
  // launch (the history, if any, committed in place); others hash, then gather.
  const bool fused_rows = !f32 && !host && ntok > 0 && ntok <= kHashGatherMaxTokens &&
                          (hist_out == nullptr || desc->seq == 1);
  if (fused_rows) {
    err = engram_launch_hash_gather_e4m3(a, params->token_map, ids, desc->batch, desc->seq,
                                         hist_in, hist_out, (const uint8_t *)table,
                                         desc->table_rows, (uint16_t *)e, stream);
    if (err != hipSuccess) return hip_status(err);
  } else {
    err = engram_launch_hash(a, params->token_map, ids, desc->batch, desc->seq, hist_in,
                             hist_out, row_ids, stream);
    if (err != hipSuccess) return hip_status(err);
    if (ntok == 0) {
      // An empty chunk still passes the convolution's history on.
      if (conv != nullptr)
        err = engram_launch_short_conv(f32, make_conv_args(conv), ids, hash_rule(params),
                                       nullptr, nullptr, h, desc->batch, desc->seq, desc->hc,
                                       desc->dim, stream);
      return hip_status(err);
    }
    err = f32 ? engram_launch_gather_f32((const float *)table, desc->table_rows, desc->row_dim,
                                         row_ids, ntok * S, (float *)e, stream)
              : engram_launch_gather_e4m3((const uint8_t *)table, desc->table_rows, row_ids,
                                          ntok * S, (uint16_t *)e, host, stream);
    if (err != hipSuccess) return hip_status(err);
  }
  // Calls that fill the CUs with whole 256 x 256 tiles take the key side of the
  // gate into the projection's epilogue: the keys never reach HBM. With the
  // convolution branch the gate then leaves its statistics to the branch.
  bool sums = false;
  if (!f32 && desc->dim % 256 == 0) {
    err = engram_gemm_bf16_whole_tiles(ntok, out_dim, in_dim, &sums);
    if (err != hipSuccess) return hip_status(err);
  }
  if (sums) {
    err = engram_launch_fold_gate_weights(q_w, k_w, qk_w, desc->hc, desc->dim, stream);
    if (err == hipSuccess)
      err = engram_launch_gemm_bf16_sums((const uint16_t *)e, (const uint16_t *)wkv, ldw,
                                         (const uint16_t *)h, qk_w, (uint16_t *)kv, ntok,
                                         desc->hc, desc->dim, in_dim, stream);
    if (err == hipSuccess)
      err = engram_launch_gate_sums(ids, hash_rule(params), kv, h, gate_out,
                                    conv != nullptr ? stats : nullptr, ntok, desc->hc, desc->dim,
                                    desc->eps, desc->gate_clamp, desc->gate_mode, stream);
    if (err != hipSuccess || conv == nullptr) return hip_status(err);
    return hip_status(engram_launch_short_conv(false, make_conv_args(conv), ids, hash_rule(params),
                                               kv, stats, h, desc->batch, desc->seq, desc->hc,
                                               desc->dim, stream));
  }
  err = f32 ? engram_launch_gemm_f32((const float *)e, (const float *)wkv, ldw, (float *)kv,
                                     ntok, out_dim, in_dim, stream)
            : engram_launch_gemm_bf16((const uint16_t *)e, (const uint16_t *)wkv, ldw,
                                      (uint16_t *)kv, ntok, out_dim, in_dim, gemm_ws,
                                      gemm_ws_bytes, stream);
  if (err != hipSuccess) return hip_status(err);
  const bool fold = ntok >= kFoldMinTokens;
  if (fold) err = engram_launch_fold_gate_weights(q_w, k_w, qk_w, desc->hc, desc->dim, stream);
  if (err != hipSuccess) return hip_status(err);
  err = engram_launch_gate(f32, ids, hash_rule(params), kv, fold ? qk_w : q_w,
                           fold ? nullptr : k_w, h, gate_out, conv != nullptr ? stats : nullptr,
                           ntok, desc->hc, desc->dim, desc->eps, desc->gate_clamp,
                           desc->gate_mode, stream);
  if (err != hipSuccess || conv == nullptr) return hip_status(err);
  err = engram_launch_short_conv(f32, make_conv_args(conv), ids, hash_rule(params), kv, stats, h,
                                 desc->batch, desc->seq, desc->hc, desc->dim, stream);
  return hip_status(err);
}

}  // namespace

extern "C" {

int engram_forward(const engram_hash_params *params, const engram_forward_desc *desc,
                   const int32_t *ids, const int32_t *hist_in, int32_t *hist_out,
                   const void *table, const void *wkv, const float *q_w, const float *k_w,
                   void *h, float *gate_out, void *workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  return forward_impl(params, desc, nullptr, ids, hist_in, hist_out, table, wkv, q_w, k_w, h,
                      gate_out, workspace, workspace_bytes, stream);
}

size_t engram_forward_conv_workspace_size(const engram_hash_params *params,
                                          const engram_forward_desc *desc) {
  const size_t base = engram_forward_workspace_size(params, desc);
  return base == 0 ? 0 : base + gate_conv_workspace(desc);
}

int engram_forward_conv(const engram_hash_params *params, const engram_forward_desc *desc,
                        const engram_short_conv *conv, const int32_t *ids,
                        const int32_t *hist_in, int32_t *hist_out, const void *table,
                        const void *wkv, const float *q_w, const float *k_w, void *h,
                        float *gate_out, void *workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  if (conv == nullptr) return ENGRAM_EINVAL;
  return forward_impl(params, desc, conv, ids, hist_in, hist_out, table, wkv, q_w, k_w, h,
                      gate_out, workspace, workspace_bytes, stream);
}



size_t engram_forward_mx_workspace_size(const engram_hash_params *params,
                                        const engram_forward_desc *desc) {
  if (check_hash_params(params) != ENGRAM_OK || check_desc(desc) != ENGRAM_OK) return 0;
  if (desc->row_format != ENGRAM_ROW_E4M3_E8M0_264) return 0;
  const int64_t ntok = desc->batch * desc->seq;
  const int32_t S = (params->max_ngram - 1) * params->heads;
  const int64_t out_dim = (int64_t)(desc->hc + 1) * desc->dim;
  return align256((size_t)ntok * S * 8) + align256((size_t)ntok * S * ENGRAM_ROW_DIM_E4M3) +
         align256((size_t)ntok * S * 8) + align256((size_t)ntok * out_dim * 2) +
         folded_scales_bytes(desc) + engram_project_mx_workspace_size(ntok, S, out_dim);
}

int engram_forward_mx(const engram_hash_params *params, const engram_forward_desc *desc,
                      const int32_t *ids, const int32_t *hist_in, int32_t *hist_out,
                      const void *table, const void *w_codes, const void *w_scales,
                      const float *q_w, const float *k_w, void *h, float *gate_out,
                      void *workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = check_hash_params(params);
  if (rc != ENGRAM_OK) return rc;
  rc = check_desc(desc);
  if (rc != ENGRAM_OK) return rc;
  if (desc->row_format != ENGRAM_ROW_E4M3_E8M0_264) return ENGRAM_EINVAL;
  if (total_rows(params) > desc->table_rows) return ENGRAM_EPRIMES;
  const int64_t ntok = desc->batch * desc->seq;
  const int32_t S = (params->max_ngram - 1) * params->heads;
  const int64_t out_dim = (int64_t)(desc->hc + 1) * desc->dim;
  if (ntok > INT32_MAX) return ENGRAM_ESHAPE;
  if (!bf16_projection_shape_ok(ntok, (int64_t)S * ENGRAM_ROW_DIM_E4M3, out_dim))
    return ENGRAM_ESHAPE;
  bool host = false;
  if (ntok > 0) {
    if (ids == nullptr || table == nullptr || w_codes == nullptr || w_scales == nullptr ||
        q_w == nullptr || k_w == nullptr || h == nullptr)
      return ENGRAM_EINVAL;
    if (!aligned(ids, 4) || !aligned(table, 8) || !aligned(w_codes, 16) ||
        !aligned(w_scales, 4) || !aligned(q_w, 16) || !aligned(k_w, 16) || !aligned(h, 16) ||
        !aligned(gate_out, 4))
      return ENGRAM_EINVAL;
    const size_t need = engram_forward_mx_workspace_size(params, desc);
    if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256))
      return ENGRAM_EWORKSPACE;
    if ((rc = resolve_table(table, desc->table_rows, &table, &host)) != ENGRAM_OK) return rc;
  }
  if (!aligned(hist_in, 4) || !aligned(hist_out, 4)) return ENGRAM_EINVAL;

  char *ws = (char *)workspace;
  int64_t *row_ids = (int64_t *)ws;
  uint8_t *e_codes = (uint8_t *)(ws + align256((size_t)ntok * S * 8));
  uint8_t *e_scales = e_codes + align256((size_t)ntok * S * ENGRAM_ROW_DIM_E4M3);
  uint16_t *kv = (uint16_t *)(e_scales + align256((size_t)ntok * S * 8));
  float *qk_w = (float *)((char *)kv + align256((size_t)ntok * out_dim * 2));
  char *gemm_ws = (char *)qk_w + folded_scales_bytes(desc);
  const size_t gemm_ws_bytes = workspace_bytes - (size_t)(gemm_ws - ws);

  const EngramHashArgs a = make_hash_args(params, 1);
  hipError_t err = hipSuccess;
  // Decode-sized calls on an HBM table form and split each token's rows in one
  // launch, as engram_forward does; others hash, then gather.
  if (!host && ntok > 0 && ntok <= kHashGatherMaxTokens &&
      (hist_out == nullptr || desc->seq == 1)) {
    err = engram_launch_hash_gather_mx(a, params->token_map, ids, desc->batch, desc->seq,
                                       hist_in, hist_out, (const uint8_t *)table,
                                       desc->table_rows, e_codes, e_scales, stream);
    if (err != hipSuccess) return hip_status(err);
  } else {
    err = engram_launch_hash(a, params->token_map, ids, desc->batch, desc->seq, hist_in,
                             hist_out, row_ids, stream);
    if (err != hipSuccess || ntok == 0) return hip_status(err);
    err = engram_launch_gather_mx((const uint8_t *)table, desc->table_rows, row_ids, ntok * S,
                                  e_codes, e_scales, host, stream);
    if (err != hipSuccess) return hip_status(err);
  }
  // As in engram_forward: whole tiles take the key side of the gate into the
  // projection's epilogue.
  bool sums = false;
  if (desc->dim % 256 == 0) {
    err = engram_gemm_mx_whole_tiles(ntok, out_dim, S, &sums);
    if (err != hipSuccess) return hip_status(err);
  }
  if (sums) {
    err = engram_launch_fold_gate_weights(q_w, k_w, qk_w, desc->hc, desc->dim, stream);
    if (err == hipSuccess)
      err = engram_launch_gemm_mx_sums((const uint8_t *)w_codes, (const uint8_t *)w_scales,
                                       e_codes, e_scales, S, (const uint16_t *)h, qk_w, kv, ntok,
                                       desc->hc, desc->dim, stream);
    if (err == hipSuccess)
      err = engram_launch_gate_sums(ids, hash_rule(params), kv, h, gate_out, nullptr, ntok,
                                    desc->hc, desc->dim, desc->eps, desc->gate_clamp,
                                    desc->gate_mode, stream);
    return hip_status(err);
  }
  err = engram_launch_gemm_mx((const uint8_t *)w_codes, (const uint8_t *)w_scales, e_codes,
                              e_scales, S, kv, ntok, out_dim, gemm_ws, gemm_ws_bytes, stream);
  if (err != hipSuccess) return hip_status(err);
  const bool fold = ntok >= kFoldMinTokens;
  if (fold) err = engram_launch_fold_gate_weights(q_w, k_w, qk_w, desc->hc, desc->dim, stream);
  if (err != hipSuccess) return hip_status(err);
  err = engram_launch_gate(false, ids, hash_rule(params), kv, fold ? qk_w : q_w,
                           fold ? nullptr : k_w, h, gate_out, nullptr, ntok, desc->hc,
                           desc->dim, desc->eps, desc->gate_clamp, desc->gate_mode, stream);
  return hip_status(err);
}

}  // extern "C"

// ---- engram_forward_static: the layer with no workspace argument ----------------
// The scratch of engram_forward (row ids, e, kv, folded gate scales, the
// projection's split-K partials) lives in this file-scope array instead of a
// caller's buffer. Every GPU the library runs on holds its own copy for the life
// of the process. In host code `scratch` names a host-side stand-in, not a
// device address: host code only ever uses the address hipGetSymbolAddress
// returns for the current device, kept per device below.
static __device__ __align__(256) unsigned char scratch[ENGRAM_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on the stream's device, looked up once per
// device with that device current. The stream must belong to the current device.
int static_scratch(hipStream_t stream, void **out) {
  int dev = -1, sdev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  e = hipStreamGetDevice(stream, &sdev);
  if (e != hipSuccess) return hip_status(e);
  if (dev != sdev || dev < 0 || dev >= kMaxScratchDevices) return ENGRAM_EINVAL;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) return hip_status(e == hipSuccess ? hipErrorUnknown : e);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ENGRAM_OK;
}

}  // namespace

extern "C" {

size_t engram_forward_static_max_bytes(void) { return ENGRAM_STATIC_SCRATCH_BYTES; }

int engram_forward_static(const engram_hash_params *params, const engram_forward_desc *desc,
                          const int32_t *ids, const int32_t *hist_in, int32_t *hist_out,
                          const void *table, const void *wkv, const float *q_w,
                          const float *k_w, void *h, float *gate_out, hipStream_t stream) {
  int rc = check_hash_params(params);
  if (rc != ENGRAM_OK) return rc;
  rc = check_desc(desc);
  if (rc != ENGRAM_OK) return rc;
  if (forward_base_bytes(params, desc) > (size_t)ENGRAM_STATIC_SCRATCH_BYTES)
    return ENGRAM_ESCRATCH;
  void *ws = nullptr;
  if ((rc = static_scratch(stream, &ws)) != ENGRAM_OK) return rc;
  // Nothing in the scratch has to start at zero: every kernel writes what a later
  // one reads (the split-K fixup reads only the partial tiles of this call).
  return forward_impl(params, desc, nullptr, ids, hist_in, hist_out, table, wkv, q_w, k_w, h,
                      gate_out, ws, ENGRAM_STATIC_SCRATCH_BYTES, stream,
                      /*gemm_ws_optional=*/true);
}

}  // extern "C"

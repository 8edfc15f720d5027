// Host side of the libtpla C ABI: argument checks, split planning and
// kernel dispatch.  Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "tpla.h"
#include "tpla_internal.h"

namespace {

thread_local char g_err[512] = "";

tpla_status fail(tpla_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

tpla_status ok() {
  g_err[0] = '\0';
  return TPLA_OK;
}

tpla_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(TPLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool valid_dtype(tpla_dtype d) { return d == TPLA_FP32 || d == TPLA_BF16; }
bool is_pow2(int64_t n) { return n > 0 && (n & (n - 1)) == 0; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Compute units of the current device, cached per device id.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

tpla_status device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev >= 0 && dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) {
      *cus = cached;
      return TPLA_OK;
    }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_status(e, "hipDeviceGetAttribute");
  if (n <= 0) n = 1;
  if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
  *cus = n;
  return TPLA_OK;
}

constexpr int64_t kMaxGenericSmem = 65536;

int64_t generic_smem(int d_s, int d_r) {
  return static_cast<int64_t>(sizeof(float)) * (16LL * (d_s + d_r) + 8LL * (d_s + d_r) + 8LL * d_s + 8 * 16 + 8 * 3);
}

enum class Path { kGeneric, kMfma, kStream };

bool mfma_operands_ok(const tpla_decode_args* a) {
  if (a->dtype != TPLA_BF16) return false;
  if (!aligned16(a->q_latent) || !aligned16(a->cache)) return false;
  if ((a->q_latent_stride_b | a->q_latent_stride_h) % 8 != 0) return false;
  if (a->d_r > 0) {
    if (!aligned16(a->q_rope)) return false;
    if ((a->q_rope_stride_b | a->q_rope_stride_h) % 8 != 0) return false;
  }
  return true;
}

Path decode_path(const tpla_decode_args* a) {
  if (!mfma_operands_ok(a)) return Path::kGeneric;
  if (tpla::decode_latsplit_supported(a->heads, a->d_s, a->d_r, a->block_size)) return Path::kStream;
  if (tpla::decode_mfma_supported(a->heads, a->d_s, a->d_r)) return Path::kMfma;
  return Path::kGeneric;
}

bool use_mfma(const tpla_decode_args* a) { return decode_path(a) != Path::kGeneric; }

tpla_status check_decode(const tpla_decode_args* a) {
  if (a == nullptr) return fail(TPLA_ERR_NULL, "args is NULL");
  if (a->batch < 1 || a->heads < 1 || a->d_s < 1 || a->d_r < 0)
    return fail(TPLA_ERR_SHAPE, "batch, heads, d_s must be >= 1 and d_r >= 0");
  if (a->block_size < 1 || a->num_blocks < 1 || a->max_blocks_per_seq < 1)
    return fail(TPLA_ERR_SHAPE, "block_size, num_blocks, max_blocks_per_seq must be >= 1");
  if (a->max_seq_len < 0 ||
      static_cast<int64_t>(a->max_seq_len) >
          static_cast<int64_t>(a->max_blocks_per_seq) * a->block_size)
    return fail(TPLA_ERR_SHAPE, "max_seq_len must be in [0, max_blocks_per_seq*block_size]");
  if (!valid_dtype(a->dtype) || !valid_dtype(a->out_dtype))
    return fail(TPLA_ERR_DTYPE, "dtype/out_dtype must be TPLA_FP32 or TPLA_BF16");
  if (!(a->scale == a->scale) || std::isinf(a->scale))
    return fail(TPLA_ERR_SHAPE, "scale must be finite");
  if (a->q_latent == nullptr || a->cache == nullptr || a->block_table == nullptr ||
      a->seq_lens == nullptr || a->out == nullptr)
    return fail(TPLA_ERR_NULL, "q_latent, cache, block_table, seq_lens and out are required");
  if (a->d_r > 0 && a->q_rope == nullptr) return fail(TPLA_ERR_NULL, "q_rope is NULL with d_r > 0");
  if (a->num_splits < 0) return fail(TPLA_ERR_SHAPE, "num_splits must be >= 0");
  if (a->q_latent_stride_h < a->d_s || a->q_latent_stride_b < 0 || a->q_rope_stride_b < 0 ||
      (a->d_r > 0 && a->q_rope_stride_h < a->d_r) ||
      a->out_stride_h < a->d_s || a->out_stride_b < 0)
    return fail(TPLA_ERR_SHAPE, "query/output head strides must cover a row");
  // A bf16 shape that a matrix-core kernel serves needs that kernel's
  // operand alignment: the float32 kernel would run it some 400x slower
  // (39 ms against 0.1 ms on the 16 x 32K-token shard), so refuse instead.
  if (a->dtype == TPLA_BF16 && !mfma_operands_ok(a) &&
      (tpla::decode_latsplit_supported(a->heads, a->d_s, a->d_r, a->block_size) ||
       tpla::decode_mfma_supported(a->heads, a->d_s, a->d_r)))
    return fail(TPLA_ERR_ALIGN,
                "bf16 decode of this shape runs on the matrix cores, which need q_latent, "
                "q_rope and cache 16-byte aligned and query strides that are multiples of 8");
  if (!use_mfma(a) && generic_smem(a->d_s, a->d_r) > kMaxGenericSmem)
    return fail(TPLA_ERR_UNSUPPORTED,
                "d_s=%d d_r=%d has no bf16 matrix-core kernel and exceeds the float32 "
                "kernel's LDS limit",
                a->d_s, a->d_r);
  return TPLA_OK;
}

struct Plan {
  int splits;
  int chunk;
  // The roles kernel cuts the work into units on the device (unit_map.h):
  // automatic calls target one unit per CU, explicit ones take `chunk`.
  bool units;
  int unit_target;
  int max_units;
  size_t ws_o_off;       // split outputs
  size_t ws_o_bytes;
  size_t lse_off;
  size_t table_off;      // unit table [batch][2] int32 (units only)
  size_t ws_bytes;
};

size_t round256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

// cus_given > 0: plan for a device with that many CUs (no device query).
tpla_status plan_decode(const tpla_decode_args* a, Plan* pl, int cus_given = 0) {
  const int maxlen = a->max_seq_len;
  int want = a->num_splits;
  int cus = cus_given;
  if (want == 0 && cus <= 0) {
    const tpla_status st = device_cus(&cus);
    if (st != TPLA_OK) return st;
  }
  if (want == 0) {
    int64_t groups = a->batch;
    int per_cu = 2;
    const Path path = decode_path(a);
    if (path == Path::kStream) {
      groups *= a->heads / tpla::decode_latsplit_heads_per_group(a->heads, a->d_s);
      per_cu = tpla::decode_latsplit_groups_per_cu(a->heads, a->d_s);
    } else if (path == Path::kMfma) {
      groups *= a->heads / (32 * (a->heads % 128 == 0 ? 4 : (a->heads % 64 == 0 ? 2 : 1)));
      per_cu = tpla::decode_mfma_groups_per_cu(a->heads, a->d_s, a->d_r);
    } else {
      groups *= (a->heads + 7) / 8;
    }
    const int64_t target = static_cast<int64_t>(cus) * per_cu;
    want = static_cast<int>(std::max<int64_t>(1, (target + groups - 1) / groups));
  }
  const int max_tiles = std::max(1, (maxlen + 63) / 64);
  want = std::min(want, max_tiles);
  if (decode_path(a) == Path::kStream &&
      tpla::decode_latsplit_supported(a->heads, a->d_s, a->d_r, a->block_size)) {
    // a split must fit the kernel's LDS table of tiles
    const int cap = tpla::decode_latsplit_max_chunk();
    want = std::max(want, static_cast<int>((static_cast<int64_t>(maxlen) + cap - 1) / cap));
  }
  const int tiles_per = (max_tiles + want - 1) / want;
  pl->chunk = tiles_per * 64;
  pl->splits = std::max(1, (maxlen + pl->chunk - 1) / pl->chunk);
  pl->units = decode_path(a) == Path::kStream &&
              tpla::decode_roles_supported(a->heads, a->d_s, a->d_r, a->block_size);
  pl->unit_target = 0;
  pl->max_units = 0;
  size_t rows = static_cast<size_t>(pl->splits) * a->batch * a->heads;
  if (pl->units) {
    const int cap = tpla::decode_roles_max_tiles();
    if (a->num_splits == 0) {
      // one unit per CU; more only where a sequence needs more than the
      // largest unit's tiles (or the batch has more sequences than CUs)
      pl->unit_target =
          std::max(1, cus / (a->heads / tpla::decode_roles_heads_per_group(a->heads, a->d_s)));
      pl->max_units = std::max<int64_t>(
          pl->unit_target, static_cast<int64_t>(a->batch) * ((max_tiles + cap - 1) / cap));
    } else {
      pl->max_units = pl->splits * a->batch;
    }
    rows = static_cast<size_t>(pl->max_units) * a->heads;
  }
  pl->ws_o_off = 0;
  pl->ws_o_bytes = round256(rows * a->d_s * sizeof(float));
  pl->lse_off = pl->ws_o_off + pl->ws_o_bytes;
  pl->table_off = pl->lse_off + round256(rows * sizeof(float));
  pl->ws_bytes = pl->table_off + (pl->units ? round256(static_cast<size_t>(a->batch) * 8) : 0);
  return TPLA_OK;
}

// Cost of one streaming-kernel launch with `splits` splits of `chunk`
// tokens, in tile units: units in the kernel's order (split fastest, then
// head group, then sequence), unit u on XCD u / per_xcd as the kernel maps
// them, in-order list scheduling onto the XCD's CU slots; a non-empty unit
// costs its tiles plus a fixed start and finish, an empty one nearly
// nothing.  Used only to pick a split count from host-side lengths.
double stream_launch_cost(const int32_t* lens, int batch, int hg, int max_len, int splits, int chunk,
                          int cus, int per_cu) {
  constexpr double kFixed = 6.0;     // start-up + tail, in tile steps
  const int64_t n_units = static_cast<int64_t>(splits) * batch * hg;
  const int64_t per_xcd = (n_units + 7) / 8;
  const int slots = std::max(1, cus / 8) * per_cu;
  double worst = 0.0;
  std::vector<double> load(static_cast<size_t>(slots));
  for (int x = 0; x < 8; ++x) {
    std::fill(load.begin(), load.end(), 0.0);
    for (int64_t u = x * per_xcd; u < std::min<int64_t>((x + 1) * per_xcd, n_units); ++u) {
      const int split = static_cast<int>(u % splits);
      const int b = static_cast<int>(u / splits / hg);
      const int L = std::max(0, std::min(lens[b], max_len));
      const int t = std::max(0, std::min(L, (split + 1) * chunk) - split * chunk);
      const double c = t > 0 ? (t + 63) / 64 + kFixed : 0.02;
      auto it = std::min_element(load.begin(), load.end());
      *it += c;
    }
    worst = std::max(worst, *std::max_element(load.begin(), load.end()));
  }
  return worst;
}

// The split suggestion for a device of `cus` CUs (<= 0: query the current
// device).
tpla_status suggest_splits(const tpla_decode_args* args, const int32_t* seq_lens_host, int cus,
                           int32_t* num_splits) {
  if (num_splits == nullptr || seq_lens_host == nullptr)
    return fail(TPLA_ERR_NULL, "seq_lens_host and num_splits are required");
  tpla_status st = check_decode(args);
  if (st != TPLA_OK) return st;
  if (cus <= 0) {
    st = device_cus(&cus);
    if (st != TPLA_OK) return st;
  }
  tpla_decode_args a = *args;
  a.num_splits = 0;
  Plan pl;
  st = plan_decode(&a, &pl, cus);
  if (st != TPLA_OK) return st;
  if (decode_path(&a) != Path::kStream) {
    *num_splits = pl.splits;
    return ok();
  }
  if (pl.units) {
    // the automatic plan balances units over the lengths on the device
    *num_splits = 0;
    return ok();
  }
  const int hg = a.heads / tpla::decode_latsplit_heads_per_group(a.heads, a.d_s);
  const int per_cu = tpla::decode_latsplit_groups_per_cu(a.heads, a.d_s);
  const int max_tiles = std::max(1, (a.max_seq_len + 63) / 64);
  const int cap_tiles = tpla::decode_latsplit_max_chunk() / 64;   // the kernel's tile table
  int best = pl.splits;
  double best_cost = 1e300;
  for (int tiles_per = 1; tiles_per <= std::min(max_tiles, cap_tiles); ++tiles_per) {
    const int splits = (max_tiles + tiles_per - 1) / tiles_per;
    if (tiles_per > 1 && (max_tiles + tiles_per - 2) / (tiles_per - 1) == splits) continue;  // same split count
    const double c = stream_launch_cost(seq_lens_host, a.batch, hg, a.max_seq_len, splits,
                                        tiles_per * 64, cus, per_cu);
    if (c < best_cost - 1e-9 || (c < best_cost + 1e-9 && splits < best)) {
      best_cost = c;
      best = splits;
    }
  }
  *num_splits = best;
  return ok();
}

}  // namespace

extern "C" {

tpla_status tpla_decode_suggest_splits(const tpla_decode_args* args, const int32_t* seq_lens_host,
                                       int32_t* num_splits) {
  return suggest_splits(args, seq_lens_host, 0, num_splits);
}

tpla_status tpla_decode_suggest_splits_cus(const tpla_decode_args* args,
                                           const int32_t* seq_lens_host, int32_t cus,
                                           int32_t* num_splits) {
  if (cus < 1) return fail(TPLA_ERR_SHAPE, "cus must be >= 1 (got %d)", cus);
  return suggest_splits(args, seq_lens_host, cus, num_splits);
}

const char* tpla_status_string(int32_t s) {
  switch (s) {
    case TPLA_OK: return "ok";
    case TPLA_ERR_NULL: return "null pointer";
    case TPLA_ERR_SHAPE: return "bad shape or size";
    case TPLA_ERR_ALIGN: return "bad alignment";
    case TPLA_ERR_DTYPE: return "unsupported dtype";
    case TPLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case TPLA_ERR_WORKSPACE: return "workspace missing or too small";
    case TPLA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* tpla_last_error(void) { return g_err; }

int32_t tpla_version(void) { return 400; }

tpla_status tpla_hadamard_latent(const void* x, tpla_dtype x_dtype, int64_t x_row_stride, void* y,
                                 tpla_dtype y_dtype, int64_t y_row_stride, int64_t rows, int32_t n,
                                 void* stream) {
  if (!valid_dtype(x_dtype) || !valid_dtype(y_dtype))
    return fail(TPLA_ERR_DTYPE, "x_dtype/y_dtype must be TPLA_FP32 or TPLA_BF16");
  if (!is_pow2(n) || n > 4096) return fail(TPLA_ERR_SHAPE, "n=%d must be a power of two <= 4096", n);
  if (rows < 0) return fail(TPLA_ERR_SHAPE, "rows must be >= 0");
  if (x_row_stride < n || y_row_stride < n)
    return fail(TPLA_ERR_SHAPE, "row strides must be >= n");
  if (rows == 0) return ok();
  if (x == nullptr || y == nullptr) return fail(TPLA_ERR_NULL, "x and y are required");
  return hip_status(tpla::launch_hadamard(x, x_dtype == TPLA_BF16, x_row_stride, y,
                                          y_dtype == TPLA_BF16, y_row_stride, rows, n,
                                          static_cast<hipStream_t>(stream)),
                    "hadamard launch");
}

tpla_status tpla_append_kv(void* cache, tpla_dtype cache_dtype, int32_t num_blocks,
                           int32_t block_size, int32_t d_s, int32_t d_r,
                           const int32_t* block_table, int32_t max_blocks_per_seq, int32_t batch,
                           const int32_t* row_seq, const int32_t* row_pos, int32_t n_rows,
                           const void* latent, int64_t latent_row_stride, const void* rope,
                           int64_t rope_row_stride, tpla_dtype src_dtype, void* stream) {
  if (!valid_dtype(cache_dtype) || !valid_dtype(src_dtype))
    return fail(TPLA_ERR_DTYPE, "cache_dtype/src_dtype must be TPLA_FP32 or TPLA_BF16");
  if (num_blocks < 1 || block_size < 1 || d_s < 1 || d_r < 0 || max_blocks_per_seq < 1 ||
      batch < 1 || n_rows < 0)
    return fail(TPLA_ERR_SHAPE, "non-positive size");
  if (latent_row_stride < d_s || (d_r > 0 && rope_row_stride < d_r))
    return fail(TPLA_ERR_SHAPE, "source row strides must cover a row");
  if (n_rows == 0) return ok();
  if (cache == nullptr || block_table == nullptr || row_seq == nullptr || row_pos == nullptr ||
      latent == nullptr || (d_r > 0 && rope == nullptr))
    return fail(TPLA_ERR_NULL, "cache, block_table, row_seq, row_pos, latent (and rope) are required");
  return hip_status(
      tpla::launch_append(cache, cache_dtype == TPLA_BF16, num_blocks, block_size, d_s, d_r,
                          block_table, max_blocks_per_seq, batch, row_seq, row_pos, n_rows, latent,
                          latent_row_stride, rope, rope_row_stride, src_dtype == TPLA_BF16,
                          static_cast<hipStream_t>(stream)),
      "append launch");
}

tpla_status tpla_rotate_append(const tpla_rotate_append_args* a, void* stream) {
  if (a == nullptr) return fail(TPLA_ERR_NULL, "args is NULL");
  if (!valid_dtype(a->q_dtype) || !valid_dtype(a->q_out_dtype) || !valid_dtype(a->src_dtype) ||
      !valid_dtype(a->cache_dtype))
    return fail(TPLA_ERR_DTYPE, "dtypes must be TPLA_FP32 or TPLA_BF16");
  const int n = a->n;
  if (!is_pow2(n) || n < 64 || n > 4096)
    return fail(TPLA_ERR_SHAPE, "n=%d must be a power of two in [64, 4096]", n);
  if (a->q_rows < 0 || a->n_rows < 0) return fail(TPLA_ERR_SHAPE, "q_rows and n_rows must be >= 0");
  if (a->n_caches < 0 || a->n_caches > tpla::kMaxTp)
    return fail(TPLA_ERR_SHAPE, "n_caches must be in [0, %d]", tpla::kMaxTp);
  if (a->latent_norm < TPLA_NORM_NONE || a->latent_norm > TPLA_NORM_SLICE)
    return fail(TPLA_ERR_SHAPE, "latent_norm=%d is not a TPLA_NORM_* value", a->latent_norm);
  if (a->latent_norm != TPLA_NORM_NONE && !(std::isfinite(a->norm_eps) && a->norm_eps > 0.f))
    return fail(TPLA_ERR_SHAPE, "norm_eps must be a positive finite number");
  if (a->latent_norm == TPLA_NORM_SLICE && (a->d_s < 1 || a->d_s > n))
    return fail(TPLA_ERR_SHAPE, "slice norm: d_s=%d must be in [1, n=%d]", a->d_s, n);
  if (a->latent_norm == TPLA_NORM_SLICE && (!is_pow2(a->d_s) || a->d_s < n / 64))
    return fail(TPLA_ERR_UNSUPPORTED, "slice norm needs d_s a power of two >= n/64, got %d", a->d_s);
  if (a->q_rows > 0) {
    if (a->q == nullptr || a->q_out == nullptr) return fail(TPLA_ERR_NULL, "q and q_out are required");
    if (a->q_row_stride < n || a->q_out_row_stride < n)
      return fail(TPLA_ERR_SHAPE, "query row strides must be >= n");
  }
  if (a->n_rows > 0) {
    if (a->latent == nullptr) return fail(TPLA_ERR_NULL, "latent is required");
    if (a->latent_row_stride < n || (a->latent_out != nullptr && a->latent_out_row_stride < n))
      return fail(TPLA_ERR_SHAPE, "latent row strides must be >= n");
    if (a->n_caches > 0) {
      if (a->num_blocks < 1 || a->block_size < 1 || a->d_s < 1 || a->d_r < 0 ||
          a->max_blocks_per_seq < 1 || a->batch < 1)
        return fail(TPLA_ERR_SHAPE, "non-positive cache size");
      if (a->first_shard < 0 ||
          static_cast<int64_t>(a->first_shard + a->n_caches) * a->d_s > n)
        return fail(TPLA_ERR_SHAPE, "shards %d..%d of width %d exceed n=%d", a->first_shard,
                    a->first_shard + a->n_caches - 1, a->d_s, n);
      if (a->d_r > 0 && (a->rope == nullptr || a->rope_row_stride < a->d_r))
        return fail(a->rope == nullptr ? TPLA_ERR_NULL : TPLA_ERR_SHAPE,
                    "rope is required with a row stride >= d_r");
      if (a->caches == nullptr || a->block_table == nullptr || a->row_seq == nullptr ||
          a->row_pos == nullptr)
        return fail(TPLA_ERR_NULL, "caches, block_table, row_seq and row_pos are required");
      for (int c = 0; c < a->n_caches; ++c)
        if (a->caches[c] == nullptr) return fail(TPLA_ERR_NULL, "caches[%d] is NULL", c);
    }
  }
  if (a->q_rows == 0 && a->n_rows == 0) return ok();
  tpla::RotateAppendParams p{};
  p.q = a->q;
  p.qs = a->q_row_stride;
  p.q_out = a->q_out;
  p.qos = a->q_out_row_stride;
  p.q_rows = a->q_rows;
  p.q_bf16 = a->q_dtype == TPLA_BF16;
  p.q_out_bf16 = a->q_out_dtype == TPLA_BF16;
  p.lat = a->latent;
  p.ls = a->latent_row_stride;
  p.rope = a->rope;
  p.rs = a->rope_row_stride;
  p.lat_out = a->latent_out;
  p.los = a->latent_out_row_stride;
  p.lat_bf16 = a->src_dtype == TPLA_BF16;
  p.n_rows = a->n_rows;
  p.row_seq = a->row_seq;
  p.row_pos = a->row_pos;
  p.n_caches = a->n_rows > 0 ? a->n_caches : 0;
  for (int c = 0; c < p.n_caches; ++c) p.caches.p[c] = a->caches[c];
  p.first_shard = a->first_shard;
  p.cache_bf16 = a->cache_dtype == TPLA_BF16;
  p.num_blocks = a->num_blocks;
  p.block_size = a->block_size;
  p.d_s = a->d_s;
  p.d_r = a->d_r;
  p.max_blocks = a->max_blocks_per_seq;
  p.batch = a->batch;
  p.bt = a->block_table;
  p.norm = a->latent_norm;
  p.norm_eps = a->norm_eps;
  return hip_status(tpla::launch_rotate_append(p, n, static_cast<hipStream_t>(stream)),
                    "rotate/append launch");
}

tpla_status tpla_decode_workspace_size(const tpla_decode_args* args, size_t* bytes) {
  if (bytes == nullptr) return fail(TPLA_ERR_NULL, "bytes is NULL");
  tpla_status st = check_decode(args);
  if (st != TPLA_OK) return st;
  Plan pl;
  st = plan_decode(args, &pl);
  if (st != TPLA_OK) return st;
  *bytes = pl.ws_bytes;
  return ok();
}

}  // extern "C"

// Scratch of tpla_decode_shard_noalloc: one copy per device, held until the
// process ends.  Host code uses only the address hipGetSymbolAddress gives
// for the current device (the array's name is a host-side stand-in).
constexpr size_t kNoAllocScratchBytes = size_t{64} << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

// The decode and merge launches of a checked, planned call whose split
// outputs go to `workspace` (at least pl.ws_bytes, 256-byte aligned).
tpla_status launch_planned_decode(const tpla_decode_args* a, const Plan& pl, void* workspace,
                                  void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);

  tpla::DecodeParams p{};
  p.batch = a->batch;
  p.heads = a->heads;
  p.d_s = a->d_s;
  p.d_r = a->d_r;
  p.block_size = a->block_size;
  p.num_blocks = a->num_blocks;
  p.max_blocks = a->max_blocks_per_seq;
  p.max_seq_len = a->max_seq_len;
  p.num_splits = pl.splits;
  p.chunk = pl.chunk;
  p.scale_log2 = a->scale * 1.4426950408889634f;
  p.q_latent = a->q_latent;
  p.qls_b = a->q_latent_stride_b;
  p.qls_h = a->q_latent_stride_h;
  p.q_rope = a->q_rope;
  p.qrs_b = a->q_rope_stride_b;
  p.qrs_h = a->q_rope_stride_h;
  p.cache = a->cache;
  p.block_table = a->block_table;
  p.seq_lens = a->seq_lens;
  char* const ws = static_cast<char*>(workspace);
  p.ws_o = reinterpret_cast<float*>(ws + pl.ws_o_off);
  p.ws_lse = reinterpret_cast<float*>(ws + pl.lse_off);
  p.unit_target = pl.unit_target;
  p.max_units = pl.max_units;
  p.unit_table = pl.units ? reinterpret_cast<int32_t*>(ws + pl.table_off) : nullptr;

  tpla::MergeParams m{};
  m.splits = pl.units ? pl.max_units : pl.splits;
  m.unit_table = p.unit_table;
  m.batch = a->batch;
  m.heads = a->heads;
  m.d_s = a->d_s;
  m.ws_o = p.ws_o;
  m.ws_lse = p.ws_lse;
  m.blk_cols = (decode_path(a) == Path::kStream &&
                tpla::decode_latsplit_supported(a->heads, a->d_s, a->d_r, a->block_size))
                   ? tpla::decode_latsplit_partial_block()
                   : 0;
  m.out = a->out;
  m.out_bf16 = a->out_dtype == TPLA_BF16;
  m.out_sb = a->out_stride_b;
  m.out_sh = a->out_stride_h;
  m.lse = a->lse;

  hipError_t e;
  switch (decode_path(a)) {
    case Path::kStream: e = tpla::launch_decode_latsplit(p, s); break;
    case Path::kMfma: e = tpla::launch_decode_mfma(p, s); break;
    default: e = tpla::launch_decode_generic(p, a->dtype == TPLA_BF16, s); break;
  }
  if (e != hipSuccess) return hip_status(e, "decode launch");
  return hip_status(tpla::launch_merge(m, s), "merge launch");
}

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device.
tpla_status scratch_address(void** ptr_out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(TPLA_ERR_UNSUPPORTED, "device %d is past the %d devices the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) return fail(TPLA_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *ptr_out = g_scratch_ptr[dev];
  return TPLA_OK;
}

}  // namespace

extern "C" {

tpla_status tpla_decode_shard(const tpla_decode_args* a, void* workspace, size_t workspace_bytes,
                              void* stream) {
  tpla_status st = check_decode(a);
  if (st != TPLA_OK) return st;
  Plan pl;
  st = plan_decode(a, &pl);
  if (st != TPLA_OK) return st;
  if (workspace == nullptr || workspace_bytes < pl.ws_bytes)
    return fail(TPLA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", pl.ws_bytes,
                workspace == nullptr ? static_cast<size_t>(0) : workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(TPLA_ERR_ALIGN, "workspace must be 256-byte aligned");
  return launch_planned_decode(a, pl, workspace, stream);
}

tpla_status tpla_decode_shard_noalloc(const tpla_decode_args* a, void* stream) {
  tpla_status st = check_decode(a);
  if (st != TPLA_OK) return st;
  Plan pl;
  st = plan_decode(a, &pl);
  if (st != TPLA_OK) return st;
  if (pl.ws_bytes > kNoAllocScratchBytes)
    return fail(TPLA_ERR_WORKSPACE,
                "this call needs %zu bytes of split outputs; the library's static scratch holds %zu "
                "(fewer splits, sequences or heads per call fit)",
                pl.ws_bytes, kNoAllocScratchBytes);
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != TPLA_OK) return st;
  return launch_planned_decode(a, pl, ws, stream);
}

size_t tpla_decode_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

tpla_status tpla_mla_prefill(const tpla_prefill_args* a, void* stream) {
  if (a == nullptr) return fail(TPLA_ERR_NULL, "args is NULL");
  if (a->batch < 1 || a->heads < 1 || a->max_len < 0)
    return fail(TPLA_ERR_SHAPE, "batch and heads must be >= 1 and max_len >= 0");
  if (a->d_c != 512 || a->d_r != 64)
    return fail(TPLA_ERR_UNSUPPORTED, "prefill needs d_c = 512 and d_r = 64 (got %d, %d)", a->d_c,
                a->d_r);
  if (a->dtype != TPLA_BF16) return fail(TPLA_ERR_DTYPE, "prefill inputs must be TPLA_BF16");
  if (!valid_dtype(a->out_dtype)) return fail(TPLA_ERR_DTYPE, "out_dtype must be TPLA_FP32 or TPLA_BF16");
  if (!(a->scale == a->scale) || std::isinf(a->scale)) return fail(TPLA_ERR_SHAPE, "scale must be finite");
  if (a->q_latent == nullptr || a->q_rope == nullptr || a->kv == nullptr || a->seq_lens == nullptr ||
      a->out == nullptr)
    return fail(TPLA_ERR_NULL, "q_latent, q_rope, kv, seq_lens and out are required");
  const int64_t d = a->d_c + a->d_r;
  if (a->q_latent_stride_h < a->d_c || a->q_rope_stride_h < a->d_r || a->out_stride_h < a->d_c ||
      a->kv_stride_t < d || a->kv_stride_t >= (int64_t{1} << 26) || a->q_latent_stride_b < 0 ||
      a->q_latent_stride_t < 0 || a->q_rope_stride_b < 0 || a->q_rope_stride_t < 0 ||
      a->kv_stride_b < 0 || a->out_stride_b < 0 || a->out_stride_t < 0)
    return fail(TPLA_ERR_SHAPE, "strides must cover a row (kv_stride_t in [d_c + d_r, 2^26))");
  if (static_cast<int64_t>(a->max_len) * a->heads > (int64_t{1} << 36))
    return fail(TPLA_ERR_SHAPE, "max_len * heads too large");
  if (!aligned16(a->q_latent) || !aligned16(a->q_rope) || !aligned16(a->kv) || !aligned16(a->out) ||
      ((a->q_latent_stride_b | a->q_latent_stride_t | a->q_latent_stride_h | a->q_rope_stride_b |
        a->q_rope_stride_t | a->q_rope_stride_h | a->kv_stride_b | a->kv_stride_t) % 8) != 0 ||
      ((a->out_stride_b | a->out_stride_t | a->out_stride_h) % 4) != 0)
    return fail(TPLA_ERR_ALIGN,
                "q_latent, q_rope, kv and out must be 16-byte aligned; query and kv strides multiples "
                "of 8 elements, out strides multiples of 4");
  if (a->max_len == 0) return ok();
  tpla::PrefillParams p{};
  p.batch = a->batch;
  p.heads = a->heads;
  p.max_len = a->max_len;
  p.scale_log2 = a->scale * 1.4426950408889634f;
  p.q_latent = a->q_latent;
  p.ql_b = a->q_latent_stride_b;
  p.ql_s = a->q_latent_stride_t;
  p.ql_h = a->q_latent_stride_h;
  p.q_rope = a->q_rope;
  p.qr_b = a->q_rope_stride_b;
  p.qr_s = a->q_rope_stride_t;
  p.qr_h = a->q_rope_stride_h;
  p.kv = a->kv;
  p.kv_b = a->kv_stride_b;
  p.kv_s = a->kv_stride_t;
  p.seq_lens = a->seq_lens;
  p.out = a->out;
  p.out_bf16 = a->out_dtype == TPLA_BF16;
  p.o_b = a->out_stride_b;
  p.o_s = a->out_stride_t;
  p.o_h = a->out_stride_h;
  p.lse = a->lse;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(tpla::prefill_roles_supported(p.heads, p.kv_s) ? tpla::launch_prefill_roles(p, s)
                                                                    : tpla::launch_mla_prefill(p, s),
                    "prefill launch");
}

tpla_status tpla_up_project(const void* o, tpla_dtype o_dtype, int64_t o_stride_b,
                            int64_t o_stride_h, const void* w, tpla_dtype w_dtype,
                            int64_t w_stride_h, int64_t w_stride_v, void* y, tpla_dtype y_dtype,
                            int64_t y_stride_b, int64_t y_stride_h, int32_t batch, int32_t heads,
                            int32_t d_s, int32_t d_v, int32_t accumulate, void* stream) {
  if (!valid_dtype(o_dtype) || !valid_dtype(w_dtype) || !valid_dtype(y_dtype))
    return fail(TPLA_ERR_DTYPE, "dtypes must be TPLA_FP32 or TPLA_BF16");
  if (batch < 1 || heads < 1 || d_s < 1 || d_v < 1)
    return fail(TPLA_ERR_SHAPE, "batch, heads, d_s, d_v must be >= 1");
  if (heads > 65535) return fail(TPLA_ERR_SHAPE, "heads=%d exceeds 65535", heads);
  if (batch > 65535 * 32) return fail(TPLA_ERR_SHAPE, "batch=%d exceeds %d", batch, 65535 * 32);
  if (o_stride_h < d_s || w_stride_v < d_s || w_stride_h < static_cast<int64_t>(d_v) * w_stride_v ||
      y_stride_h < d_v || o_stride_b < 0 || y_stride_b < 0)
    return fail(TPLA_ERR_SHAPE, "strides must cover a row");
  if (o == nullptr || w == nullptr || y == nullptr) return fail(TPLA_ERR_NULL, "o, w and y are required");
  tpla::UpProjectParams p{};
  p.o = o;
  p.o_sb = o_stride_b;
  p.o_sh = o_stride_h;
  p.w = w;
  p.w_sh = w_stride_h;
  p.w_sv = w_stride_v;
  p.y = y;
  p.y_sb = y_stride_b;
  p.y_sh = y_stride_h;
  p.batch = batch;
  p.heads = heads;
  p.d_s = d_s;
  p.d_v = d_v;
  p.accumulate = accumulate != 0;
  return hip_status(tpla::launch_up_project(p, o_dtype == TPLA_BF16, w_dtype == TPLA_BF16,
                                            y_dtype == TPLA_BF16, static_cast<hipStream_t>(stream)),
                    "up-projection launch");
}

tpla_status tpla_combine_shards(const void* const* partials, tpla_dtype part_dtype, int32_t tp,
                                int32_t batch, int32_t heads, int32_t d_s, void* out,
                                tpla_dtype out_dtype, int32_t accumulate, void* stream) {
  if (!valid_dtype(part_dtype) || !valid_dtype(out_dtype))
    return fail(TPLA_ERR_DTYPE, "part_dtype/out_dtype must be TPLA_FP32 or TPLA_BF16");
  if (tp < 1 || tp > tpla::kMaxTp) return fail(TPLA_ERR_SHAPE, "tp=%d must be in [1, 16]", tp);
  if (batch < 1 || heads < 1 || d_s < 1) return fail(TPLA_ERR_SHAPE, "non-positive size");
  if (partials == nullptr || out == nullptr) return fail(TPLA_ERR_NULL, "partials and out are required");
  tpla::PartPtrs pp{};
  for (int g = 0; g < tp; ++g) {
    if (partials[g] == nullptr) return fail(TPLA_ERR_NULL, "partials[%d] is NULL", g);
    pp.p[g] = partials[g];
  }
  return hip_status(tpla::launch_combine(pp, part_dtype == TPLA_BF16, tp, batch, heads, d_s, out,
                                         out_dtype == TPLA_BF16, accumulate != 0,
                                         static_cast<hipStream_t>(stream)),
                    "combine launch");
}

}  // extern "C"

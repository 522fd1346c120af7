// nm_api.hip -- the C ABI declared in include/nm.h: argument checks and dispatch.
//
// Every check runs on the host before any HIP call, so a rejected call touches
// neither the device nor the outputs.  The global state is a per-device record of
// whether the device is a gfx950, filled on first use, and the per-device address of
// the static scratch buffer behind nm_perm_gains_static, looked up on first use.
#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/nm.h"
#include "nm_launch.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = unsupported device
std::atomic<int> g_device_ok[kMaxDevices];

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A pointer may be NULL only when the array it addresses is empty.
bool missing(const void* p, int64_t count) { return p == nullptr && count > 0; }

int meta_bits_of(int m) { return m == 2 ? 1 : m == 4 ? 2 : m == 8 ? 3 : -1; }

int elem_bytes(nm_dtype dt) { return dt == NM_F32 ? 4 : (dt == NM_I8 || dt == NM_FP8) ? 1 : 2; }

// Element types of W for the selection and the products; NM_I32 is an output type only.
bool valid_dtype(int dt) {
  return dt == NM_F32 || dt == NM_F16 || dt == NM_BF16 || dt == NM_I8 || dt == NM_FP8;
}
bool float_dtype(int dt) { return dt == NM_F32 || dt == NM_F16 || dt == NM_BF16; }

// The blocked layout stores a lane's 16 elements of a block as whole 32-bit words of values:
// for byte elements (int8, fp8), 16 N / M bytes must divide by 4.
bool blocked_pattern_ok(nm_dtype dt, int n, int m) {
  return elem_bytes(dt) != 1 || (16 * n / m) % 4 == 0;
}

nm_status check_pattern(int n, int m) {
  if (meta_bits_of(m) < 0 || n < 1 || n > m) return NM_ERR_PATTERN;
  return NM_OK;
}

nm_status check_shape(int64_t R, int64_t K, int m) {
  if (R < 0 || K < 0 || K % m != 0) return NM_ERR_SHAPE;
  // below 2^36 elements (128 GiB of 16-bit W) every launch of the element-wise passes has
  // fewer than 2^32 work-items: their fast kernels give each work-item at least 16 elements,
  // and the per-group fallbacks loop over a capped grid
  if (R > 0 && K >= ((int64_t)1 << 36) / R + ((((int64_t)1 << 36) % R) != 0)) return NM_ERR_SHAPE;
  return NM_OK;
}

nm_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NM_ERR_DEVICE;
  int state = g_device_ok[dev].load(std::memory_order_acquire);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return NM_ERR_DEVICE;
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_device_ok[dev].store(state, std::memory_order_release);
  }
  return state == 1 ? NM_OK : NM_ERR_DEVICE;
}

// Do the byte ranges [a, a + a_bytes) and [b, b + b_bytes) share a byte?
bool overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return a_bytes > 0 && b_bytes > 0 && x < y + (uintptr_t)b_bytes && y < x + (uintptr_t)a_bytes;
}
bool overlaps(const void* a, const void* b, int64_t bytes) { return overlaps(a, bytes, b, bytes); }

nm_status from_hip(hipError_t e) { return e == hipSuccess ? NM_OK : NM_ERR_DEVICE; }

// NM_LAYOUT_BLOCKED cuts K into steps of 64: each step then holds a whole number of
// groups (M divides 64) and of metadata bytes (64 N / M fields of log2(M) bits).
nm_status check_layout(int layout, int64_t K) {
  if (layout == NM_LAYOUT_ROWS) return NM_OK;
  if (layout == NM_LAYOUT_BLOCKED && K % 64 == 0) return NM_OK;
  return NM_ERR_LAYOUT;
}

int64_t padded_rows(int64_t R, int layout) { return layout == NM_LAYOUT_BLOCKED ? (R + 15) / 16 * 16 : R; }

// Bytes of metadata per row: the row's whole words (ROWS) or its K/64 step slices (BLOCKED).
int64_t meta_row_bytes(int64_t K, int n, int m, int layout) {
  const int64_t bits = (K / m) * n * meta_bits_of(m);
  return layout == NM_LAYOUT_BLOCKED ? bits / 8 : (bits + 31) / 32 * 4;
}

}  // namespace

extern "C" {

int nm_abi_version(void) { return NM_ABI_VERSION; }

const char* nm_status_str(nm_status s) {
  switch (s) {
    case NM_OK: return "ok";
    case NM_ERR_NULL: return "null pointer";
    case NM_ERR_SHAPE: return "bad shape (negative size, K not a multiple of M, or R*K >= 2^36)";
    case NM_ERR_PATTERN: return "bad N:M pattern (need 1 <= N <= M, M in {2,4,8})";
    case NM_ERR_DTYPE: return "bad dtype (unknown, or output neither input dtype nor fp32)";
    case NM_ERR_ALIGN: return "pointer not 16-byte aligned";
    case NM_ERR_UNSUPPORTED: return "unsupported combination";
    case NM_ERR_DEVICE: return "device error (no gfx950 device, or launch failed)";
    case NM_ERR_LAYOUT: return "bad layout (unknown, or blocked layout with K not a multiple of 64)";
    case NM_ERR_ALIAS: return "an output overlaps an input it may not replace";
    case NM_ERR_SCRATCH: return "the call needs more than the library's static scratch buffer";
  }
  return "unknown status";
}

size_t nm_values_bytes(int64_t R, int64_t K, int n, int m, nm_dtype dt, nm_layout layout) {
  if (!valid_dtype(dt) || check_pattern(n, m) != NM_OK || check_shape(R, K, m) != NM_OK ||
      check_layout(layout, K) != NM_OK)
    return 0;
  if (layout == NM_LAYOUT_BLOCKED && !blocked_pattern_ok(dt, n, m)) return 0;
  return (size_t)(padded_rows(R, layout) * (K / m * n) * elem_bytes(dt));
}

size_t nm_meta_bytes(int64_t R, int64_t K, int n, int m, nm_layout layout) {
  if (check_pattern(n, m) != NM_OK || check_shape(R, K, m) != NM_OK ||
      check_layout(layout, K) != NM_OK)
    return 0;
  return (size_t)(padded_rows(R, layout) * meta_row_bytes(K, n, m, layout));
}

int64_t nm_check_meta(const uint32_t* meta_host, int64_t R, int64_t K, int n, int m,
                      nm_layout layout) {
  if (check_pattern(n, m) != NM_OK || check_shape(R, K, m) != NM_OK ||
      check_layout(layout, K) != NM_OK)
    return -2;
  if (R * K == 0) return -1;
  if (meta_host == nullptr) return -2;
  const int b = meta_bits_of(m);
  const int64_t G = K / m, row_bits = G * n * b;
  const uint8_t* bytes = reinterpret_cast<const uint8_t*>(meta_host);
  const int64_t row_bytes = meta_row_bytes(K, n, m, layout);
  std::vector<uint8_t> row((size_t)row_bytes + 2);  // + 2: a field read may look past the end
  for (int64_t r = 0; r < R; ++r) {
    if (layout == NM_LAYOUT_ROWS) {
      std::memcpy(row.data(), bytes + r * row_bytes, (size_t)row_bytes);
    } else {  // the row's slice of every 64-wide step, from block (r / 16, s)
      const int64_t S = K / 64, B = row_bytes / S;
      for (int64_t st = 0; st < S; ++st)
        std::memcpy(row.data() + st * B, bytes + (((r / 16) * S + st) * 16 + r % 16) * B, (size_t)B);
    }
    row[row_bytes] = row[row_bytes + 1] = 0;
    auto field = [&](int64_t f) {  // b bits at bit f * b, least significant first
      const int64_t bit = f * b;
      const uint32_t v = row[bit / 8] | (uint32_t)row[bit / 8 + 1] << 8;
      return (int)((v >> (bit % 8)) & ((1u << b) - 1u));
    };
    for (int64_t g = 0; g < G; ++g) {
      int prev = -1;
      for (int j = 0; j < n; ++j) {
        const int p = field(g * n + j);
        if (p <= prev) return r * G + g;
        prev = p;
      }
    }
    for (int64_t bit = row_bits; bit < row_bytes * 8; ++bit)
      if ((row[bit / 8] >> (bit % 8)) & 1u) return r * G + G - 1;
  }
  return -1;
}

int64_t nm_meta_words_per_row(int64_t K, int n, int m) {
  if (check_pattern(n, m) != NM_OK || K < 0 || K % m != 0) return -1;
  return ((K / m) * n * meta_bits_of(m) + 31) / 32;
}

nm_status nm_mask(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m, uint8_t* mask,
                  nm_stream_t stream) {
  if (!valid_dtype(dt)) return NM_ERR_DTYPE;
  nm_status st = check_pattern(n, m);
  if (st != NM_OK) return st;
  if ((st = check_shape(R, K, m)) != NM_OK) return st;
  if (missing(W, R * K) || missing(mask, R * K)) return NM_ERR_NULL;
  if (R * K == 0) return NM_OK;
  if (!aligned16(W) || !aligned16(mask)) return NM_ERR_ALIGN;
  if (overlaps(mask, R * K, W, R * K * elem_bytes(dt))) return NM_ERR_ALIAS;
  if ((st = check_device()) != NM_OK) return st;
  return from_hip(nm::launch_select(W, (int)dt, R, K, n, m, false, nullptr, nullptr, mask,
                                    static_cast<hipStream_t>(stream)));
}

nm_status nm_compress(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m,
                      nm_layout layout, void* values, uint32_t* meta, nm_stream_t stream) {
  if (!valid_dtype(dt)) return NM_ERR_DTYPE;
  nm_status st = check_pattern(n, m);
  if (st != NM_OK) return st;
  if ((st = check_shape(R, K, m)) != NM_OK) return st;
  if ((st = check_layout(layout, K)) != NM_OK) return st;
  if (layout == NM_LAYOUT_BLOCKED && !blocked_pattern_ok(dt, n, m)) return NM_ERR_UNSUPPORTED;
  if (missing(W, R * K) || missing(values, R * K) || missing(meta, R * K)) return NM_ERR_NULL;
  if (R * K == 0) return NM_OK;
  if (!aligned16(W) || !aligned16(values) || !aligned16(meta)) return NM_ERR_ALIGN;
  {
    const int64_t w_bytes = R * K * elem_bytes(dt);
    const int64_t v_bytes = (int64_t)nm_values_bytes(R, K, n, m, dt, layout);
    const int64_t m_bytes = (int64_t)nm_meta_bytes(R, K, n, m, layout);
    if (overlaps(values, v_bytes, W, w_bytes) || overlaps(meta, m_bytes, W, w_bytes) ||
        overlaps(values, v_bytes, meta, m_bytes))
      return NM_ERR_ALIAS;
  }
  if ((st = check_device()) != NM_OK) return st;
  return from_hip(nm::launch_select(W, (int)dt, R, K, n, m, layout == NM_LAYOUT_BLOCKED,
                                    values, meta, nullptr, static_cast<hipStream_t>(stream)));
}

nm_status nm_mask_compress(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m,
                           nm_layout layout, uint8_t* mask, void* values, uint32_t* meta,
                           nm_stream_t stream) {
  if (!valid_dtype(dt)) return NM_ERR_DTYPE;
  nm_status st = check_pattern(n, m);
  if (st != NM_OK) return st;
  if ((st = check_shape(R, K, m)) != NM_OK) return st;
  if ((st = check_layout(layout, K)) != NM_OK) return st;
  if (layout == NM_LAYOUT_BLOCKED && !blocked_pattern_ok(dt, n, m)) return NM_ERR_UNSUPPORTED;
  if (missing(W, R * K) || missing(mask, R * K) || missing(values, R * K) ||
      missing(meta, R * K))
    return NM_ERR_NULL;
  if (R * K == 0) return NM_OK;
  if (!aligned16(W) || !aligned16(mask) || !aligned16(values) || !aligned16(meta))
    return NM_ERR_ALIGN;
  const int64_t w_bytes = R * K * elem_bytes(dt), mask_bytes = R * K;
  const int64_t v_bytes = (int64_t)nm_values_bytes(R, K, n, m, dt, layout);
  const int64_t m_bytes = (int64_t)nm_meta_bytes(R, K, n, m, layout);
  if (overlaps(mask, mask_bytes, W, w_bytes) || overlaps(values, v_bytes, W, w_bytes) ||
      overlaps(meta, m_bytes, W, w_bytes) || overlaps(mask, mask_bytes, values, v_bytes) ||
      overlaps(mask, mask_bytes, meta, m_bytes) || overlaps(values, v_bytes, meta, m_bytes))
    return NM_ERR_ALIAS;
  if ((st = check_device()) != NM_OK) return st;
  return from_hip(nm::launch_select(W, (int)dt, R, K, n, m, layout == NM_LAYOUT_BLOCKED, values,
                                    meta, mask, static_cast<hipStream_t>(stream)));
}

nm_status nm_decompress(const void* values, const uint32_t* meta, nm_dtype dt, int64_t R,
                        int64_t K, int n, int m, nm_layout layout, void* W_out,
                        nm_stream_t stream) {
  if (!valid_dtype(dt)) return NM_ERR_DTYPE;
  nm_status st = check_pattern(n, m);
  if (st != NM_OK) return st;
  if ((st = check_shape(R, K, m)) != NM_OK) return st;
  if ((st = check_layout(layout, K)) != NM_OK) return st;
  if (layout == NM_LAYOUT_BLOCKED && !blocked_pattern_ok(dt, n, m)) return NM_ERR_UNSUPPORTED;
  if (missing(values, R * K) || missing(meta, R * K) || missing(W_out, R * K)) return NM_ERR_NULL;
  if (R * K == 0) return NM_OK;
  if (!aligned16(values) || !aligned16(meta) || !aligned16(W_out)) return NM_ERR_ALIGN;
  {
    const int64_t w_bytes = R * K * elem_bytes(dt);
    if (overlaps(W_out, w_bytes, values, (int64_t)nm_values_bytes(R, K, n, m, dt, layout)) ||
        overlaps(W_out, w_bytes, meta, (int64_t)nm_meta_bytes(R, K, n, m, layout)))
      return NM_ERR_ALIAS;
  }
  if ((st = check_device()) != NM_OK) return st;
  return from_hip(nm::launch_decompress(values, meta, elem_bytes(dt), R, K, n, m,
                                        layout == NM_LAYOUT_BLOCKED, W_out,
                                        static_cast<hipStream_t>(stream)));
}

nm_status nm_spmm(const void* values, const uint32_t* meta, int64_t R, int64_t K, int n, int m,
                  nm_layout layout, const void* X, int64_t T, nm_dtype dt, void* Y,
                  nm_dtype y_dt, nm_stream_t stream) {
  if (dt == NM_I8) {
    if (y_dt != NM_I32) return NM_ERR_DTYPE;
  } else if (dt == NM_FP8) {
    if (y_dt != NM_F32 && y_dt != NM_BF16) return NM_ERR_DTYPE;
  } else if (!float_dtype(dt) || !float_dtype(y_dt) || (y_dt != dt && y_dt != NM_F32)) {
    return NM_ERR_DTYPE;
  }
  nm_status st = check_pattern(n, m);
  if (st != NM_OK) return st;
  if ((st = check_shape(R, K, m)) != NM_OK) return st;
  if (dt == NM_I8 && K >= (int64_t)1 << 17) return NM_ERR_SHAPE;  // int32 sums stay exact
  if ((st = check_layout(layout, K)) != NM_OK) return st;
  if (layout == NM_LAYOUT_BLOCKED && !blocked_pattern_ok(dt, n, m)) return NM_ERR_UNSUPPORTED;
  if (T < 0 || (K > 0 && T > ((int64_t)1 << 40) / K) || (R > 0 && T > ((int64_t)1 << 40) / R))
    return NM_ERR_SHAPE;
  if (missing(values, R * K) || missing(meta, R * K) || missing(X, K * T) || missing(Y, R * T))
    return NM_ERR_NULL;
  if (R * T == 0) return NM_OK;
  if (!aligned16(values) || !aligned16(meta) || !aligned16(X) || !aligned16(Y)) return NM_ERR_ALIGN;
  {
    // Y is written while other workgroups still read values, meta and X
    const int64_t y_bytes = R * T * ((y_dt == NM_F32 || y_dt == NM_I32) ? 4 : 2);
    if (overlaps(Y, y_bytes, X, K * T * elem_bytes(dt)) ||
        overlaps(Y, y_bytes, values, (int64_t)nm_values_bytes(R, K, n, m, dt, layout)) ||
        overlaps(Y, y_bytes, meta, (int64_t)nm_meta_bytes(R, K, n, m, layout)))
      return NM_ERR_ALIAS;
  }
  if ((st = check_device()) != NM_OK) return st;
  return from_hip(nm::launch_spmm(values, meta, R, K, n, m, layout == NM_LAYOUT_BLOCKED, X, T,
                                  (int)dt, Y, (int)y_dt, static_cast<hipStream_t>(stream)));
}

nm_status nm_tmask(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m, uint8_t* mask,
                   nm_stream_t stream) {
  if (!float_dtype(dt)) return NM_ERR_DTYPE;
  nm_status st = check_pattern(n, m);
  if (st != NM_OK) return st;
  if ((st = check_shape(R, K, m)) != NM_OK) return st;
  if (R % m != 0) return NM_ERR_SHAPE;
  if (missing(W, R * K) || missing(mask, R * K)) return NM_ERR_NULL;
  if (R * K == 0) return NM_OK;
  if (overlaps(W, R * K * elem_bytes(dt), mask, R * K)) return NM_ERR_ALIAS;
  if (!aligned16(W) || !aligned16(mask)) return NM_ERR_ALIGN;
  if ((st = check_device()) != NM_OK) return st;
  return from_hip(nm::launch_tmask(W, elem_bytes(dt), R, K, n, m, false, mask,
                                   static_cast<hipStream_t>(stream)));
}

nm_status nm_tprune(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m, void* W_out,
                    nm_stream_t stream) {
  if (!float_dtype(dt)) return NM_ERR_DTYPE;
  nm_status st = check_pattern(n, m);
  if (st != NM_OK) return st;
  if ((st = check_shape(R, K, m)) != NM_OK) return st;
  if (R % m != 0) return NM_ERR_SHAPE;
  if (missing(W, R * K) || missing(W_out, R * K)) return NM_ERR_NULL;
  if (R * K == 0) return NM_OK;
  if (W_out != W && overlaps(W, W_out, R * K * elem_bytes(dt))) return NM_ERR_ALIAS;
  if (!aligned16(W) || !aligned16(W_out)) return NM_ERR_ALIGN;
  if ((st = check_device()) != NM_OK) return st;
  return from_hip(nm::launch_tmask(W, elem_bytes(dt), R, K, n, m, true, W_out,
                                   static_cast<hipStream_t>(stream)));
}

nm_status nm_compress_t(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m,
                        nm_layout layout, void* values, uint32_t* meta, nm_stream_t stream) {
  if (!float_dtype(dt)) return NM_ERR_DTYPE;
  nm_status st = check_pattern(n, m);
  if (st != NM_OK) return st;
  if ((st = check_shape(K, R, m)) != NM_OK) return st;  // the transpose is K x R
  if ((st = check_layout(layout, R)) != NM_OK) return st;
  if (missing(W, R * K) || missing(values, R * K) || missing(meta, R * K)) return NM_ERR_NULL;
  if (R * K == 0) return NM_OK;
  const int64_t wb = R * K * elem_bytes(dt);
  if (overlaps(W, wb, values, (int64_t)nm_values_bytes(K, R, n, m, dt, layout)) ||
      overlaps(W, wb, meta, (int64_t)nm_meta_bytes(K, R, n, m, layout)))
    return NM_ERR_ALIAS;
  if (!aligned16(W) || !aligned16(values) || !aligned16(meta)) return NM_ERR_ALIGN;
  if ((st = check_device()) != NM_OK) return st;
  return from_hip(nm::launch_select_t(W, elem_bytes(dt), R, K, n, m, layout == NM_LAYOUT_BLOCKED,
                                      values, meta, static_cast<hipStream_t>(stream)));
}

nm_status nm_prune(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m, void* W_out,
                   nm_stream_t stream) {
  if (!float_dtype(dt)) return NM_ERR_DTYPE;
  nm_status st = check_pattern(n, m);
  if (st != NM_OK) return st;
  if ((st = check_shape(R, K, m)) != NM_OK) return st;
  if (missing(W, R * K) || missing(W_out, R * K)) return NM_ERR_NULL;
  if (R * K == 0) return NM_OK;
  if (W_out != W && overlaps(W, W_out, R * K * elem_bytes(dt))) return NM_ERR_ALIAS;
  if (!aligned16(W) || !aligned16(W_out)) return NM_ERR_ALIGN;
  if ((st = check_device()) != NM_OK) return st;
  return from_hip(nm::launch_prune(W, (int)dt, R, K, n, m, W_out,
                                   static_cast<hipStream_t>(stream)));
}

nm_status nm_srste_grad(const void* W, const void* G, nm_dtype dt, int64_t R, int64_t K, int n,
                        int m, float decay, void* G_out, nm_stream_t stream) {
  if (!float_dtype(dt)) return NM_ERR_DTYPE;
  nm_status st = check_pattern(n, m);
  if (st != NM_OK) return st;
  if ((st = check_shape(R, K, m)) != NM_OK) return st;
  if (missing(W, R * K) || missing(G, R * K) || missing(G_out, R * K)) return NM_ERR_NULL;
  if (R * K == 0) return NM_OK;
  const int64_t bytes = R * K * elem_bytes(dt);
  if (overlaps(W, G_out, bytes) || (G_out != G && overlaps(G, G_out, bytes))) return NM_ERR_ALIAS;
  if (!aligned16(W) || !aligned16(G) || !aligned16(G_out)) return NM_ERR_ALIGN;
  if ((st = check_device()) != NM_OK) return st;
  return from_hip(nm::launch_srste_grad(W, G, (int)dt, R, K, n, m, decay, G_out,
                                        static_cast<hipStream_t>(stream)));
}

size_t nm_perm_workspace_bytes(int64_t R, int64_t K, int n, int m) {
  if (check_pattern(n, m) != NM_OK || check_shape(R, K, m) != NM_OK) return 0;
  if (R * K >= ((int64_t)1 << 31)) return 0;
  return nm::perm_workspace_bytes(R, K, m);
}

namespace {
nm_status check_perm_args(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m,
                          const void* workspace, size_t workspace_bytes) {
  if (!valid_dtype(dt)) return NM_ERR_DTYPE;
  nm_status st = check_pattern(n, m);
  if (st != NM_OK) return st;
  if ((st = check_shape(R, K, m)) != NM_OK) return st;
  if (R * K >= ((int64_t)1 << 31)) return NM_ERR_SHAPE;  // 32-bit gather indices
  if (missing(W, R * K) || missing(workspace, R * K)) return NM_ERR_NULL;
  if (R * K > 0 && workspace_bytes < nm::perm_workspace_bytes(R, K, m)) return NM_ERR_SHAPE;
  if (!aligned16(W) || !aligned16(workspace)) return NM_ERR_ALIGN;
  return NM_OK;
}
}  // namespace

nm_status nm_perm_gains(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m,
                        const int32_t* perm, float* gain, int32_t* pick, void* workspace,
                        size_t workspace_bytes, nm_stream_t stream) {
  nm_status st = check_perm_args(W, dt, R, K, n, m, workspace, workspace_bytes);
  if (st != NM_OK) return st;
  const int64_t G = K / m;
  if (missing(perm, K) || missing(gain, G * G) || missing(pick, G * G)) return NM_ERR_NULL;
  if (R * K == 0 || G < 2) return NM_OK;
  if ((st = check_device()) != NM_OK) return st;
  return from_hip(nm::launch_perm_gains(W, (int)dt, R, K, n, m, perm, gain, pick, workspace,
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// The scratch buffer of nm_perm_gains_static.  Each device holds its own copy at its own
// address; in host code the name is only the host-side handle of the symbol, so kernels get
// the device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[NM_STATIC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on device `dev` (the current device), looked up once per
// device; nullptr if the lookup fails.
void* scratch_on(int dev) {
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

nm_status nm_perm_gains_static(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m,
                               const int32_t* perm, float* gain, int32_t* pick,
                               nm_stream_t stream) {
  if (!valid_dtype(dt)) return NM_ERR_DTYPE;
  nm_status st = check_pattern(n, m);
  if (st != NM_OK) return st;
  if ((st = check_shape(R, K, m)) != NM_OK) return st;
  if (R * K >= ((int64_t)1 << 31)) return NM_ERR_SHAPE;  // 32-bit gather indices, as nm_perm_gains
  const int64_t G = K / m;
  if (missing(W, R * K) || missing(perm, K) || missing(gain, G * G) || missing(pick, G * G))
    return NM_ERR_NULL;
  // the kernels use only the permuted fp32 copy of W: the first part of the workspace
  if ((size_t)(R * K) * 4 > NM_STATIC_SCRATCH_BYTES) return NM_ERR_SCRATCH;
  if (!aligned16(W)) return NM_ERR_ALIGN;
  if (R * K == 0 || G < 2) return NM_OK;
  if ((st = check_device()) != NM_OK) return st;
  int dev = 0, sdev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NM_ERR_DEVICE;
  if (stream != nullptr &&
      (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess || sdev != dev))
    return NM_ERR_DEVICE;
  void* ws = scratch_on(dev);
  if (ws == nullptr) return NM_ERR_DEVICE;
  return from_hip(nm::launch_perm_gains(W, (int)dt, R, K, n, m, perm, gain, pick, ws,
                                        static_cast<hipStream_t>(stream)));
}

nm_status nm_perm_search(const void* W, nm_dtype dt, int64_t R, int64_t K, int n, int m,
                         int max_rounds, int32_t* perm, int* rounds, void* workspace,
                         size_t workspace_bytes, nm_stream_t stream) {
  nm_status st = check_perm_args(W, dt, R, K, n, m, workspace, workspace_bytes);
  if (st != NM_OK) return st;
  if (missing(perm, K)) return NM_ERR_NULL;
  if (max_rounds < 0) return NM_ERR_SHAPE;
  // perm must be a permutation of 0 .. K-1
  std::vector<uint8_t> seen((size_t)K, 0);
  for (int64_t i = 0; i < K; ++i) {
    if (perm[i] < 0 || perm[i] >= K || seen[(size_t)perm[i]]) return NM_ERR_SHAPE;
    seen[(size_t)perm[i]] = 1;
  }
  if (rounds) *rounds = 0;
  if (R * K == 0 || K / m < 2 || max_rounds == 0) return NM_OK;
  if ((st = check_device()) != NM_OK) return st;
  return from_hip(nm::run_perm_search(W, (int)dt, R, K, n, m, max_rounds, perm, rounds,
                                      workspace, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// C ABI of libwpa (declared in include/wpa.h): argument checks, the window and rotation
// tables, the closed-form kept-term count, workspace sizing and kernel launches.
#include "wpa.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "wpa_internal.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = 0;
    return WPA_OK;
}

// ---- Debug mode: WPA_DEBUG set in the environment (to anything but "0"), or wpa_set_debug(1).
// An entry point then also checks, before it enqueues anything, that every device buffer it
// will touch lies inside one allocation of at least the bytes it needs, and that the
// preconditions on device-resident values hold (read back to the host after the stream
// drains); after enqueueing it waits for the stream and reports a failure there as
// WPA_ERR_HIP from the call that caused it.  All of this is host code around the launches.
std::atomic<int> g_debug{-1};

bool debug_on() {
    int v = g_debug.load(std::memory_order_relaxed);
    if (v < 0) {
        const char* e = std::getenv("WPA_DEBUG");
        v = (e && *e && std::strcmp(e, "0") != 0) ? 1 : 0;
        g_debug.store(v, std::memory_order_relaxed);
    }
    return v == 1;
}

size_t esize(int32_t dtype) { return dtype == WPA_FP32 ? 4 : 2; }

// [p, p + bytes) inside one allocation the HIP runtime knows (device, or pinned host memory)
int dbg_extent(const void* p, size_t bytes, const char* name) {
    if (!p || bytes == 0) return WPA_OK;
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess || !base) {
        (void)hipGetLastError();
        return fail(WPA_ERR_INVALID, "debug: %s (%p) is not inside an allocation of the HIP runtime",
                    name, p);
    }
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b0 = reinterpret_cast<uintptr_t>(base);
    if (a + bytes > b0 + size)
        return fail(WPA_ERR_INVALID, "debug: %s needs %zu bytes from %p, but its allocation ends %zu "
                    "bytes after it", name, bytes, p, (size_t)(b0 + size - a));
    return WPA_OK;
}

// copy n device values to the host once the stream has drained (after dbg_extent)
template <typename T>
int dbg_fetch(const T* p, size_t n, std::vector<T>* h, void* stream, const char* name) {
    h->assign(n, T{});
    if (!p || n == 0) return WPA_OK;
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = hipMemcpy(h->data(), p, n * sizeof(T), hipMemcpyDeviceToHost);
    if (e != hipSuccess)
        return fail(WPA_ERR_HIP, "debug: reading %s back: %s", name, hipGetErrorString(e));
    return WPA_OK;
}

// wait for the stream; a device-side failure becomes this call's error
int dbg_finish(void* stream, const char* what) {
    const hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(WPA_ERR_HIP, "debug: %s failed on the device: %s", what, hipGetErrorString(e));
    return ok();
}

// Debug checks of values the kernels trust: positions non-decreasing in [0, 2^31) per
// sequence; per-head rotation frequencies finite, > 0 and non-increasing per row.
int dbg_positions(const int32_t* pos, int32_t B, int64_t N, void* stream) {
    if (!pos) return WPA_OK;
    int rc = dbg_extent(pos, (size_t)B * N * 4, "positions");
    if (rc) return rc;
    std::vector<int32_t> h;
    rc = dbg_fetch(pos, (size_t)B * N, &h, stream, "positions");
    if (rc) return rc;
    for (int32_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < N; ++t) {
            const int32_t x = h[(size_t)b * N + t];
            if (x < 0) return fail(WPA_ERR_INVALID, "debug: positions[%d][%lld] = %d is negative", b, (long long)t, x);
            if (t > 0 && x < h[(size_t)b * N + t - 1])
                return fail(WPA_ERR_INVALID, "debug: positions of sequence %d decrease at %lld", b, (long long)t);
        }
    return WPA_OK;
}

int dbg_head_tables(const wpa_rope_t* rope, int32_t Hkv, int32_t d, void* stream) {
    const double* t = rope ? rope->head_inv_freq : nullptr;
    if (!t) return WPA_OK;
    int rc = dbg_extent(t, (size_t)Hkv * (d / 2) * sizeof(double), "head_inv_freq");
    if (rc) return rc;
    std::vector<double> h;
    rc = dbg_fetch(t, (size_t)Hkv * (d / 2), &h, stream, "head_inv_freq");
    if (rc) return rc;
    for (int32_t g = 0; g < Hkv; ++g)
        for (int i = 0; i < d / 2; ++i) {
            const double x = h[(size_t)g * (d / 2) + i];
            if (!(x > 0.0) || !std::isfinite(x) || (i > 0 && x > h[(size_t)g * (d / 2) + i - 1]))
                return fail(WPA_ERR_INVALID, "debug: head_inv_freq[%d][%d] = %g (rows must be finite, "
                            "> 0 and non-increasing)", g, i, x);
        }
    return WPA_OK;
}

// page-table entries of the pages that tokens [t0, t1) of sequence b reach
int dbg_pages(const std::vector<int32_t>& table, int32_t b, int32_t max_pages, int32_t page_log2,
              int32_t num_pages, int64_t t0, int64_t t1) {
    if (t1 <= t0) return WPA_OK;
    for (int64_t i = t0 >> page_log2; i <= (t1 - 1) >> page_log2; ++i) {
        const int32_t pg = table[(size_t)b * max_pages + i];
        if (pg < 0 || pg >= num_pages)
            return fail(WPA_ERR_INVALID, "debug: block_table[%d][%lld] = %d is outside [0, %d)", b,
                        (long long)i, pg, num_pages);
    }
    return WPA_OK;
}

// The decode caches (K in layout kl, V by key octets) or the page pools and, for the latter,
// the table entries of the pages that tokens [t0[b], t1[b]) of each sequence reach.
int dbg_caches(const void* kc, const void* vc, int32_t B, int64_t Lmax, int32_t Hkv, int32_t d,
               const wpa::KLayout& kl, const wpa::Paging& pg, const std::vector<int64_t>& t0,
               const std::vector<int64_t>& t1, void* stream) {
    int rc;
    if (!pg.table) {
        if ((rc = dbg_extent(kc, (size_t)B * Hkv * kl.head * 32, "k_cache")) ||
            (rc = dbg_extent(vc, (size_t)B * Hkv * ((Lmax + 7) / 8) * 8 * d * 2, "v_cache")))
            return rc;
        return WPA_OK;
    }
    const size_t page = (size_t)Hkv * d * ((size_t)1 << pg.page_log2) * 2;
    if ((rc = dbg_extent(kc, page * pg.num_pages, "k_pool")) ||
        (rc = dbg_extent(vc, page * pg.num_pages, "v_pool")) ||
        (rc = dbg_extent(pg.table, (size_t)B * pg.max_pages * 4, "block_table")))
        return rc;
    std::vector<int32_t> table;
    if ((rc = dbg_fetch(pg.table, (size_t)B * pg.max_pages, &table, stream, "block_table"))) return rc;
    for (int32_t b = 0; b < B; ++b)
        if ((rc = dbg_pages(table, b, pg.max_pages, pg.page_log2, pg.num_pages, t0[b], t1[b]))) return rc;
    return WPA_OK;
}

// alpha*lambda_i, lambda_i = 2*pi*base^(2i/d): one full rotation period of pair i
// (WavePrune original abstract: each channel keeps its first rotation period at alpha=1;
// ATFlash abstract: the distance window is proportional to the wavelength).  With a
// frequency table, lambda_i = 2*pi/theta_i.
double window_value(int d, double base, const double* inv_freq, double alpha, int i) {
    const double lam = inv_freq ? (2.0 * M_PI) / inv_freq[i]
                                : (2.0 * M_PI) * std::pow(base, (2.0 * i) / (double)d);
    return alpha * lam;
}

const double* freq_table(const wpa_rope_t* rope) { return rope ? rope->inv_freq : nullptr; }
const double* head_tables(const wpa_rope_t* rope) { return rope ? rope->head_inv_freq : nullptr; }
int interleaved(const wpa_rope_t* rope) { return rope && rope->pairs == WPA_PAIRS_INTERLEAVED; }

// The RoPE description: a known pair layout; a frequency table positive, finite and
// non-increasing (the pairs active at a distance must stay a suffix), else a base > 1.
int check_rope(int32_t d, double base, const wpa_rope_t* rope) {
    if (rope && rope->pairs != WPA_PAIRS_HALF && rope->pairs != WPA_PAIRS_INTERLEAVED)
        return fail(WPA_ERR_INVALID, "rope pairs must be WPA_PAIRS_HALF or WPA_PAIRS_INTERLEAVED");
    if (head_tables(rope)) {
        // per-kv-head tables live on the device: their values are the caller's contract
        if (freq_table(rope)) return fail(WPA_ERR_INVALID, "give inv_freq or head_inv_freq, not both");
        if (reinterpret_cast<uintptr_t>(head_tables(rope)) & 7u)
            return fail(WPA_ERR_INVALID, "head_inv_freq must be 8-byte aligned");
        return WPA_OK;
    }
    const double* f = freq_table(rope);
    if (!f) {
        if (!(base > 1.0) || !std::isfinite(base)) return fail(WPA_ERR_INVALID, "rope base must be finite and > 1");
        return WPA_OK;
    }
    for (int i = 0; i < d / 2; ++i) {
        if (!(f[i] > 0.0) || !std::isfinite(f[i]))
            return fail(WPA_ERR_UNSUPPORTED, "inv_freq[%d] = %g: rotation frequencies must be finite and > 0", i, f[i]);
        if (i > 0 && f[i] > f[i - 1])
            return fail(WPA_ERR_UNSUPPORTED, "inv_freq must be non-increasing (inv_freq[%d] > inv_freq[%d])", i, i - 1);
    }
    return WPA_OK;
}

// Integer form used by the kernels: distance D (an integer) is inside iff D <= floor(t).
int32_t window_int(double t) {
    if (!(t < (double)INT32_MAX)) return INT32_MAX;
    return (int32_t)std::floor(t);
}

// Paths that take one table for all heads only (their windows or cache layouts are fixed
// on the host, or their kernels read the launch's table).
int no_head_tables(const wpa_rope_t* rope, const char* what) {
    if (head_tables(rope))
        return fail(WPA_ERR_UNSUPPORTED, "%s takes no per-head frequency tables", what);
    return WPA_OK;
}

int check_common(int32_t d, double base, const wpa_rope_t* rope, double alpha) {
    if (d != 64 && d != 128) return fail(WPA_ERR_UNSUPPORTED, "head dim d=%d unsupported (64 or 128)", d);
    const int rc = check_rope(d, base, rope);
    if (rc) return rc;
    if (!(alpha >= 0.0)) return fail(WPA_ERR_INVALID, "alpha must be >= 0 (got %g)", alpha);
    return WPA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

void make_tables(int32_t d, double base, const wpa_rope_t* rope, double alpha, wpa::Tables* t) {
    std::memset(t, 0, sizeof *t);
    const double* f = freq_table(rope);
    for (int i = 0; i < d / 2; ++i) {
        t->W[i] = window_int(window_value(d, base, f, alpha, i));
        t->theta[i] = f ? f[i] : std::pow(base, -(2.0 * i) / (double)d);
    }
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// K rows of one (sequence, kv head) when every pair block keeps all `rows` tokens.
wpa::KLayout dense_layout(int32_t d, int64_t rows) {
    wpa::KLayout kl{};
    for (int j = 0; j < d / 16; ++j) {
        kl.off[j] = j * rows;
        kl.cap[j] = (int32_t)rows;
    }
    kl.head = (int64_t)(d / 16) * rows;
    return kl;
}

// The windowed decode cache: pair block j keeps only the keys still inside its largest
// window W = floor(cache_alpha * lambda) of its last pair (windows grow with the pair index),
// i.e. the newest W + 1 tokens, rounded up to 32 rows; a block whose window reaches the
// cache length keeps all Lmax.  In decode the query is the newest token, so a key that has
// left a block's window never re-enters it: the block's older rows can be reused (a ring).
wpa::KLayout window_layout(int32_t d, int64_t Lmax, double base, const wpa_rope_t* rope,
                           double cache_alpha) {
    wpa::KLayout kl{};
    int64_t off = 0;
    for (int j = 0; j < d / 16; ++j) {
        const double t = window_value(d, base, freq_table(rope), cache_alpha, 8 * j + 7);
        int64_t cap = Lmax;
        if (t < (double)(Lmax - 1)) cap = round_up((int64_t)std::floor(t) + 1, 32);
        if (cap > Lmax) cap = Lmax;
        kl.off[j] = off;
        kl.cap[j] = (int32_t)cap;
        off += cap;
    }
    kl.head = off;
    return kl;
}

int default_chunk(int32_t B, int64_t Lmax, int32_t Hkv) {
    // About two work items per compute unit (one round of resident workgroups: 256 CUs x
    // 2), at least 256 keys each.  Fewer, longer items stream the caches faster: measured
    // on the Llama-3.2-3B (16 x 131072) and Qwen2.5-7B (1 x 1M) decode shapes, 512 items
    // beat 4096 by 7% and 20%.
    const int64_t keys = (int64_t)B * Hkv * Lmax;
    int64_t c = 256;
    while (c < (1 << 20) && keys > 512 * c) c <<= 1;
    return (int)c;
}

// sum over integer r in [a, b] of max(0, hi(r) - lo(r) + 1) for the visible-window count,
// evaluated piecewise (each piece linear in r).  Used by the closed form below.
__int128 sum_linear(int64_t a, int64_t b, int64_t c0, int64_t c1) {
    // sum_{r=a}^{b} (c1*r + c0); requires a <= b
    const __int128 n = (__int128)b - a + 1;
    const __int128 sr = ((__int128)a + b) * n / 2;
    return (__int128)c1 * sr + (__int128)c0 * n;
}

// kept terms of one pair with integer threshold Wi (>= 0, possibly huge): queries r in
// [q0, q0+nq), keys c in [0, nk), visible iff c <= r, kept iff r - c <= Wi.
// For query r the kept keys are c in [max(0, r - Wi), min(r, nk - 1)].
__int128 pair_kept(int64_t q0, int64_t nq, int64_t nk, int64_t Wi) {
    const int64_t r_lo = q0, r_hi = q0 + nq - 1;
    // breakpoints: r = Wi (lower end leaves 0), r = nk - 1 (upper end saturates)
    int64_t cuts[4] = {r_lo, r_hi + 1, 0, 0};
    int nc = 2;
    if (Wi + 1 > r_lo && Wi + 1 <= r_hi) cuts[nc++] = Wi + 1;
    if (nk > r_lo && nk <= r_hi) cuts[nc++] = nk;
    for (int i = 0; i < nc; ++i)
        for (int j = i + 1; j < nc; ++j)
            if (cuts[j] < cuts[i]) { int64_t t = cuts[i]; cuts[i] = cuts[j]; cuts[j] = t; }
    __int128 total = 0;
    for (int s = 0; s + 1 < nc; ++s) {
        const int64_t a = cuts[s], b = cuts[s + 1] - 1;
        if (a > b) continue;
        // on [a, b] both ends are linear: lo = (a > Wi ? r - Wi : 0), hi = (a >= nk ? nk-1 : r)
        const bool lo_shift = a > Wi;
        const bool hi_sat = a >= nk;
        // count(r) = hi - lo + 1 ; may be <= 0 only if hi_sat && lo_shift and r - Wi > nk - 1
        if (hi_sat && lo_shift) {
            // count = nk - 1 - (r - Wi) + 1 = (nk + Wi) - r, positive while r < nk + Wi
            const int64_t b2 = (b < nk + Wi - 1) ? b : nk + Wi - 1;
            if (a <= b2) total += sum_linear(a, b2, nk + Wi, -1);
        } else if (hi_sat) {
            total += (__int128)nk * ((__int128)b - a + 1);          // keys 0..nk-1
        } else if (lo_shift) {
            total += (__int128)(Wi + 1) * ((__int128)b - a + 1);    // keys r-Wi..r
        } else {
            total += sum_linear(a, b, 1, 1);                         // keys 0..r
        }
    }
    return total;
}

}  // namespace

extern "C" {

const char* wpa_last_error(void) { return g_err; }

int wpa_set_debug(int32_t on) {
    const int was = debug_on() ? 1 : 0;
    if (on >= 0) g_debug.store(on ? 1 : 0, std::memory_order_relaxed);
    return was;
}

int wpa_thresholds_ex(int32_t d, double base, const wpa_rope_t* rope, double alpha, int32_t* W) {
    if (d < 2 || d > 128 || (d & 1)) return fail(WPA_ERR_INVALID, "d must be even and in [2, 128]");
    int rc = check_rope(d, base, rope);
    if (rc) return rc;
    rc = no_head_tables(rope, "wpa_thresholds_ex (host only: pass one head's table as inv_freq)");
    if (rc) return rc;
    if (!(alpha >= 0.0)) return fail(WPA_ERR_INVALID, "alpha must be >= 0");
    if (!W) return fail(WPA_ERR_INVALID, "W is null");
    for (int i = 0; i < d / 2; ++i) W[i] = window_int(window_value(d, base, freq_table(rope), alpha, i));
    return ok();
}

int wpa_thresholds(int32_t d, double base, double alpha, int32_t* W) {
    return wpa_thresholds_ex(d, base, nullptr, alpha, W);
}

int wpa_count_terms(int32_t d, double base, double alpha, int64_t n_q, int64_t q_pos0,
                    int64_t n_k, int64_t* kept, int64_t* total) {
    return wpa_count_terms_ex(d, base, nullptr, alpha, n_q, q_pos0, n_k, kept, total);
}

int wpa_count_terms_ex(int32_t d, double base, const wpa_rope_t* rope, double alpha, int64_t n_q,
                       int64_t q_pos0, int64_t n_k, int64_t* kept, int64_t* total) {
    if (d < 2 || (d & 1)) return fail(WPA_ERR_INVALID, "d must be even and >= 2");
    int rc = check_rope(d, base, rope);
    if (rc) return rc;
    rc = no_head_tables(rope, "wpa_count_terms_ex (host only: count each head with its table as inv_freq)");
    if (rc) return rc;
    if (!(alpha >= 0.0)) return fail(WPA_ERR_INVALID, "alpha must be >= 0");
    if (n_q < 0 || n_k < 0 || q_pos0 < 0) return fail(WPA_ERR_INVALID, "negative count or position");
    if (!kept || !total) return fail(WPA_ERR_INVALID, "null output pointer");
    __int128 k = 0, vis = 0;
    if (n_q > 0 && n_k > 0) {
        vis = pair_kept(q_pos0, n_q, n_k, INT64_MAX / 4);
        for (int i = 0; i < d / 2; ++i) {
            const double t = window_value(d, base, freq_table(rope), alpha, i);
            const int64_t Wi = (t < 9.0e18) ? (int64_t)std::floor(t) : INT64_MAX / 4;
            k += pair_kept(q_pos0, n_q, n_k, Wi);
        }
    }
    const __int128 tot = vis * (d / 2);
    if (tot > (__int128)INT64_MAX) return fail(WPA_ERR_INVALID, "count overflows int64");
    *kept = (int64_t)k;
    *total = (int64_t)tot;
    return ok();
}

size_t wpa_prefill_workspace_bytes(int32_t B, int64_t N, int32_t Hkv, int32_t d) {
    if (B < 1 || N < 1 || Hkv < 1 || d < 1) return 0;
    return (size_t)2 * B * Hkv * round_up(N, wpa::kTileKeys) * d * 2;
}

namespace {

int check_prefill_shape(int64_t N, int32_t B, int32_t Hkv, int32_t dtype, const int32_t* positions,
                        const void* workspace, size_t ws_bytes, int32_t d) {
    if (B < 1 || N < 1 || Hkv < 1) return fail(WPA_ERR_INVALID, "B, N, Hkv must be >= 1");
    if (N >= (int64_t)INT32_MAX - wpa::kTileKeys) return fail(WPA_ERR_INVALID, "N too large");
    if (dtype != WPA_BF16 && dtype != WPA_FP32) return fail(WPA_ERR_INVALID, "dtype must be WPA_BF16 or WPA_FP32");
    if (!workspace) return fail(WPA_ERR_INVALID, "null workspace");
    if (!aligned16(workspace)) return fail(WPA_ERR_INVALID, "workspace must be 16-byte aligned");
    if (positions && (reinterpret_cast<uintptr_t>(positions) & 3u))
        return fail(WPA_ERR_INVALID, "positions must be 4-byte aligned");
    const size_t need = wpa_prefill_workspace_bytes(B, N, Hkv, d);
    if (ws_bytes < need) return fail(WPA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    return WPA_OK;
}

}  // namespace

int wpa_prefill_prepare(const void* k, const void* v, const int32_t* positions, int32_t B,
                        int64_t N, int32_t Hkv, int32_t d, double base, int32_t dtype,
                        void* workspace, size_t ws_bytes, void* stream) {
    return wpa_prefill_prepare_ex(k, v, positions, B, N, Hkv, d, base, nullptr, dtype, workspace,
                                  ws_bytes, stream);
}

int wpa_prefill_prepare_ex(const void* k, const void* v, const int32_t* positions, int32_t B,
                           int64_t N, int32_t Hkv, int32_t d, double base, const wpa_rope_t* rope,
                           int32_t dtype, void* workspace, size_t ws_bytes, void* stream) {
    int rc = check_common(d, base, rope, 1.0);
    if (rc) return rc;
    rc = check_prefill_shape(N, B, Hkv, dtype, positions, workspace, ws_bytes, d);
    if (rc) return rc;
    if (!k || !v) return fail(WPA_ERR_INVALID, "null k or v");
    if (!aligned16(k) || !aligned16(v)) return fail(WPA_ERR_INVALID, "k and v must be 16-byte aligned");
    wpa::Tables tab;
    make_tables(d, base, rope, 1.0, &tab);
    const int64_t Np = round_up(N, wpa::kTileKeys);
    uint16_t* kp = static_cast<uint16_t*>(workspace);
    wpa::RopeParams rp{};
    rp.k = k; rp.v = v; rp.pos = positions; rp.kp = kp; rp.vout = kp + (size_t)B * Hkv * Np * d;
    rp.n = N; rp.t0 = 0; rp.ld = Np; rp.pad_to = Np; rp.kl = dense_layout(d, Np);
    rp.B = B; rp.Hkv = Hkv; rp.d = d; rp.in_f32 = dtype == WPA_FP32; rp.v_prefill = 1;
    rp.interleaved = interleaved(rope);
    rp.head_theta = head_tables(rope);
    rp.tab = &tab;
    if (debug_on()) {
        const size_t kv = (size_t)B * N * Hkv * d * esize(dtype);
        if ((rc = dbg_extent(k, kv, "k")) || (rc = dbg_extent(v, kv, "v")) ||
            (rc = dbg_extent(workspace, wpa_prefill_workspace_bytes(B, N, Hkv, d), "workspace")) ||
            (rc = dbg_positions(positions, B, N, stream)) || (rc = dbg_head_tables(rope, Hkv, d, stream)))
            return rc;
    }
    hipError_t e = wpa::launch_rope_relayout(rp, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(WPA_ERR_HIP, "rope relayout launch: %s", hipGetErrorString(e));
    if (debug_on()) return dbg_finish(stream, "prefill prepare");
    return ok();
}

int wpa_prefill_attend(const void* q, void* out, float* lse, const int32_t* positions,
                       int32_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t d, double base,
                       double alpha, float scale, int32_t dtype, int32_t out_dtype,
                       unsigned long long* term_count, const void* workspace, size_t ws_bytes,
                       void* stream) {
    return wpa_prefill_attend_ex(q, out, lse, positions, B, N, Hq, Hkv, d, base, nullptr, alpha,
                                 scale, dtype, out_dtype, term_count, workspace, ws_bytes, stream);
}

}  // extern "C"

namespace {

int attend_impl(const void* q, void* out, float* lse, const int32_t* positions, int32_t B,
                int64_t N, int32_t Hq, int32_t Hkv, int32_t d, double base,
                const wpa_rope_t* rope, double alpha, float scale, int32_t dtype,
                int32_t out_dtype, unsigned long long* term_count, const void* workspace,
                size_t ws_bytes, void* stream, const int32_t* blk_count,
                const int32_t* blk_idx, int32_t blk_max, int32_t blk_log2 = 6);

}  // namespace

extern "C" {

int wpa_prefill_attend_ex(const void* q, void* out, float* lse, const int32_t* positions,
                          int32_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t d, double base,
                          const wpa_rope_t* rope, double alpha, float scale, int32_t dtype,
                          int32_t out_dtype, unsigned long long* term_count,
                          const void* workspace, size_t ws_bytes, void* stream) {
    return attend_impl(q, out, lse, positions, B, N, Hq, Hkv, d, base, rope, alpha, scale, dtype,
                       out_dtype, term_count, workspace, ws_bytes, stream, nullptr, nullptr, 0);
}

}  // extern "C"

namespace {

int attend_impl(const void* q, void* out, float* lse, const int32_t* positions, int32_t B,
                int64_t N, int32_t Hq, int32_t Hkv, int32_t d, double base,
                const wpa_rope_t* rope, double alpha, float scale, int32_t dtype,
                int32_t out_dtype, unsigned long long* term_count, const void* workspace,
                size_t ws_bytes, void* stream, const int32_t* blk_count,
                const int32_t* blk_idx, int32_t blk_max, int32_t blk_log2) {
    int rc = check_common(d, base, rope, alpha);
    if (rc) return rc;
    rc = check_prefill_shape(N, B, Hkv, dtype, positions, workspace, ws_bytes, d);
    if (rc) return rc;
    if (Hq < 1) return fail(WPA_ERR_INVALID, "Hq must be >= 1");
    if (Hq % Hkv) return fail(WPA_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (out_dtype != WPA_BF16 && out_dtype != WPA_FP32) return fail(WPA_ERR_INVALID, "out_dtype must be WPA_BF16 or WPA_FP32");
    if (std::isnan(scale)) return fail(WPA_ERR_INVALID, "scale is NaN");
    if (!q || !out) return fail(WPA_ERR_INVALID, "null q or out");
    if (!aligned16(q) || !aligned16(out)) return fail(WPA_ERR_INVALID, "q and out must be 16-byte aligned");
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(WPA_ERR_INVALID, "lse must be 4-byte aligned");
    if (term_count && (reinterpret_cast<uintptr_t>(term_count) & 7u)) return fail(WPA_ERR_INVALID, "term_count must be 8-byte aligned");
    wpa::Tables tab;
    make_tables(d, base, rope, alpha, &tab);
    const int64_t Np = round_up(N, wpa::kTileKeys);
    const uint16_t* kp = static_cast<const uint16_t*>(workspace);
    wpa::PrefillParams pp{};
    pp.interleaved = interleaved(rope);
    pp.q = q; pp.kp = kp; pp.vt = kp + (size_t)B * Hkv * Np * d; pp.out = out; pp.lse = lse;
    pp.pos = positions; pp.counter = term_count; pp.N = N; pp.Np = Np; pp.ldk = Np; pp.B = B; pp.Hq = Hq;
    pp.Hkv = Hkv; pp.d = d; pp.in_f32 = dtype == WPA_FP32; pp.out_f32 = out_dtype == WPA_FP32;
    pp.scale = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)d));
    pp.blk_count = blk_count; pp.blk_idx = blk_idx; pp.blk_max = blk_max; pp.blk_log2 = blk_log2;
    pp.head_theta = head_tables(rope);
    pp.alpha = alpha;
    if (debug_on()) {
        const size_t qo = (size_t)B * N * Hq * d, nblk = (size_t)((N + (1 << blk_log2) - 1) >> blk_log2);
        if ((rc = dbg_extent(q, qo * esize(dtype), "q")) ||
            (rc = dbg_extent(out, qo * esize(out_dtype), "out")) ||
            (rc = dbg_extent(lse, (size_t)B * Hq * N * 4, "lse")) ||
            (rc = dbg_extent(term_count, 8, "term_count")) ||
            (rc = dbg_extent(workspace, wpa_prefill_workspace_bytes(B, N, Hkv, d), "workspace")) ||
            (rc = dbg_extent(blk_count, (size_t)B * Hq * nblk * 4, "blk_count")) ||
            (rc = dbg_extent(blk_idx, (size_t)B * Hq * nblk * (blk_max > 0 ? blk_max : 0) * 4, "blk_idx")) ||
            (rc = dbg_positions(positions, B, N, stream)) || (rc = dbg_head_tables(rope, Hkv, d, stream)))
            return rc;
    }
    hipError_t e = wpa::launch_prefill(pp, tab, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(WPA_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
    if (debug_on()) return dbg_finish(stream, "prefill attend");
    return ok();
}

}  // namespace

extern "C" {

int wpa_prefill(const void* q, const void* k, const void* v, void* out, float* lse,
                const int32_t* positions, int32_t B, int64_t N, int32_t Hq, int32_t Hkv,
                int32_t d, double base, double alpha, float scale, int32_t dtype,
                int32_t out_dtype, unsigned long long* term_count, void* workspace,
                size_t ws_bytes, void* stream) {
    return wpa_prefill_ex(q, k, v, out, lse, positions, B, N, Hq, Hkv, d, base, nullptr, alpha,
                          scale, dtype, out_dtype, term_count, workspace, ws_bytes, stream);
}

int wpa_prefill_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                   const int32_t* positions, int32_t B, int64_t N, int32_t Hq, int32_t Hkv,
                   int32_t d, double base, const wpa_rope_t* rope, double alpha, float scale,
                   int32_t dtype, int32_t out_dtype, unsigned long long* term_count,
                   void* workspace, size_t ws_bytes, void* stream) {
    // check everything before enqueueing anything
    int rc = check_common(d, base, rope, alpha);
    if (rc) return rc;
    if (B < 1 || N < 1 || Hq < 1 || Hkv < 1) return fail(WPA_ERR_INVALID, "B, N, Hq, Hkv must be >= 1");
    if (Hq % Hkv) return fail(WPA_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (std::isnan(scale)) return fail(WPA_ERR_INVALID, "scale is NaN");
    if (out_dtype != WPA_BF16 && out_dtype != WPA_FP32) return fail(WPA_ERR_INVALID, "out_dtype must be WPA_BF16 or WPA_FP32");
    if (!q || !k || !v || !out) return fail(WPA_ERR_INVALID, "null q, k, v or out");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(WPA_ERR_INVALID, "q, k, v and out must be 16-byte aligned");
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(WPA_ERR_INVALID, "lse must be 4-byte aligned");
    if (term_count && (reinterpret_cast<uintptr_t>(term_count) & 7u)) return fail(WPA_ERR_INVALID, "term_count must be 8-byte aligned");
    rc = check_prefill_shape(N, B, Hkv, dtype, positions, workspace, ws_bytes, d);
    if (rc) return rc;
    rc = wpa_prefill_prepare_ex(k, v, positions, B, N, Hkv, d, base, rope, dtype, workspace,
                                ws_bytes, stream);
    if (rc) return rc;
    return wpa_prefill_attend_ex(q, out, lse, positions, B, N, Hq, Hkv, d, base, rope, alpha, scale,
                                 dtype, out_dtype, term_count, workspace, ws_bytes, stream);
}

int wpa_prefill_sparse(const void* q, const void* k, const void* v, void* out, float* lse,
                       const int32_t* blk_count, const int32_t* blk_idx, int32_t blk_max,
                       int32_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t d, double base,
                       const wpa_rope_t* rope, double alpha, float scale, int32_t dtype,
                       int32_t out_dtype, unsigned long long* term_count, void* workspace,
                       size_t ws_bytes, void* stream) {
    return wpa_prefill_sparse_ex(q, k, v, out, lse, blk_count, blk_idx, blk_max, 64, B, N, Hq,
                                 Hkv, d, base, rope, alpha, scale, dtype, out_dtype, term_count,
                                 workspace, ws_bytes, stream);
}

// Block-sparse prefill, at token indices (positions null) or at explicit positions.  The
// blocks are always token-index blocks; the positions only move the rotation and the window.
static int sparse_impl(const void* q, const void* k, const void* v, void* out, float* lse,
                       const int32_t* blk_count, const int32_t* blk_idx, int32_t blk_max,
                       int32_t block, const int32_t* positions, int32_t B, int64_t N, int32_t Hq,
                       int32_t Hkv, int32_t d, double base, const wpa_rope_t* rope, double alpha,
                       float scale, int32_t dtype, int32_t out_dtype,
                       unsigned long long* term_count, void* workspace, size_t ws_bytes,
                       void* stream) {
    int rc = check_common(d, base, rope, alpha);
    if (rc) return rc;
    if (block < 64 || block > 1024 || (block & (block - 1)))
        return fail(WPA_ERR_INVALID, "block must be a power of two from 64 to 1024 (got %d)", block);
    const int32_t blk_log2 = __builtin_ctz((unsigned)block);
    if (B < 1 || N < 1 || Hq < 1 || Hkv < 1) return fail(WPA_ERR_INVALID, "B, N, Hq, Hkv must be >= 1");
    if (Hq % Hkv) return fail(WPA_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (N > ((int64_t)1 << 21)) return fail(WPA_ERR_UNSUPPORTED, "block-sparse prefill supports N up to 2^21 tokens");
    if (!blk_count || (blk_max > 0 && !blk_idx) || blk_max < 0)
        return fail(WPA_ERR_INVALID, "block lists: need blk_count, blk_max >= 0 and blk_idx when blk_max > 0");
    if ((reinterpret_cast<uintptr_t>(blk_count) & 3u) || (reinterpret_cast<uintptr_t>(blk_idx) & 3u))
        return fail(WPA_ERR_INVALID, "block lists must be 4-byte aligned");
    if (std::isnan(scale)) return fail(WPA_ERR_INVALID, "scale is NaN");
    if (out_dtype != WPA_BF16 && out_dtype != WPA_FP32) return fail(WPA_ERR_INVALID, "out_dtype must be WPA_BF16 or WPA_FP32");
    if (!q || !k || !v || !out) return fail(WPA_ERR_INVALID, "null q, k, v or out");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(WPA_ERR_INVALID, "q, k, v and out must be 16-byte aligned");
    rc = check_prefill_shape(N, B, Hkv, dtype, positions, workspace, ws_bytes, d);
    if (rc) return rc;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(WPA_ERR_INVALID, "lse must be 4-byte aligned");
    if (term_count && (reinterpret_cast<uintptr_t>(term_count) & 7u)) return fail(WPA_ERR_INVALID, "term_count must be 8-byte aligned");
    {
        // the lists live in LDS as bitmaps next to the kernel's tiles: check the fit before
        // anything is enqueued (at d = 128 this bounds N below 2^21)
        wpa::PrefillParams pp{};
        pp.d = d; pp.in_f32 = dtype == WPA_FP32; pp.N = N; pp.counter = term_count;
        pp.head_theta = head_tables(rope); pp.pos = positions;
        size_t need = 0, limit = 0;
        hipError_t e = wpa::prefill_sparse_lds(pp, &need, &limit);
        if (e != hipSuccess) return fail(WPA_ERR_HIP, "block-sparse LDS query: %s", hipGetErrorString(e));
        if (need > limit)
            return fail(WPA_ERR_UNSUPPORTED, "block-sparse prefill of %lld tokens at d=%d needs %zu bytes of LDS per "
                        "workgroup (limit %zu)", (long long)N, d, need, limit);
    }
    rc = wpa_prefill_prepare_ex(k, v, positions, B, N, Hkv, d, base, rope, dtype, workspace,
                                ws_bytes, stream);
    if (rc) return rc;
    return attend_impl(q, out, lse, positions, B, N, Hq, Hkv, d, base, rope, alpha, scale, dtype,
                       out_dtype, term_count, workspace, ws_bytes, stream, blk_count,
                       blk_idx ? blk_idx : blk_count, blk_max, blk_log2);
}

int wpa_prefill_sparse_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                          const int32_t* blk_count, const int32_t* blk_idx, int32_t blk_max,
                          int32_t block, int32_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t d,
                          double base, const wpa_rope_t* rope, double alpha, float scale,
                          int32_t dtype, int32_t out_dtype, unsigned long long* term_count,
                          void* workspace, size_t ws_bytes, void* stream) {
    return sparse_impl(q, k, v, out, lse, blk_count, blk_idx, blk_max, block, nullptr, B, N, Hq,
                       Hkv, d, base, rope, alpha, scale, dtype, out_dtype, term_count, workspace,
                       ws_bytes, stream);
}

int wpa_prefill_sparse_pos(const void* q, const void* k, const void* v, void* out, float* lse,
                           const int32_t* blk_count, const int32_t* blk_idx, int32_t blk_max,
                           int32_t block, const int32_t* positions, int32_t B, int64_t N,
                           int32_t Hq, int32_t Hkv, int32_t d, double base, const wpa_rope_t* rope,
                           double alpha, float scale, int32_t dtype, int32_t out_dtype,
                           unsigned long long* term_count, void* workspace, size_t ws_bytes,
                           void* stream) {
    if (!positions) return fail(WPA_ERR_INVALID, "null positions (use wpa_prefill_sparse_ex for token indices)");
    return sparse_impl(q, k, v, out, lse, blk_count, blk_idx, blk_max, block, positions, B, N, Hq,
                       Hkv, d, base, rope, alpha, scale, dtype, out_dtype, term_count, workspace,
                       ws_bytes, stream);
}

// Workspace of the prefill backward: its regions, in order, each 256-byte aligned.
struct BwdLayout {
    size_t off[11];
    size_t total;
};

BwdLayout bwd_layout(int32_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t d) {
    const int64_t Np = round_up(N, wpa::kTileKeys);
    const size_t kvh = (size_t)B * Hkv * Np * d, qh = (size_t)B * Hq * Np * d, rows = (size_t)B * Hq * Np;
    const size_t sz[11] = {kvh * 2, kvh * 2, qh * 2, qh * 2, qh * 2, rows * 4, rows * 4, qh * 4, qh * 4,
                           kvh * 2, qh * 2};
    BwdLayout L{};
    size_t at = 0;
    for (int i = 0; i < 11; ++i) {
        L.off[i] = at;
        at += (sz[i] + 255) / 256 * 256;
    }
    L.total = at;
    return L;
}

size_t wpa_prefill_backward_workspace_bytes(int32_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t d) {
    if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || d < 1) return 0;
    return bwd_layout(B, N, Hq, Hkv, d).total;
}

int wpa_prefill_backward(const void* q, const void* k, const void* v, const void* out,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv,
                         int32_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t d, double base,
                         const wpa_rope_t* rope, double alpha, float scale, int32_t dtype,
                         int32_t out_dtype, int32_t grad_dtype, void* workspace, size_t ws_bytes,
                         void* stream) {
    int rc = check_common(d, base, rope, alpha);
    if (rc) return rc;
    rc = no_head_tables(rope, "wpa_prefill_backward");
    if (rc) return rc;
    if (B < 1 || N < 1 || Hq < 1 || Hkv < 1) return fail(WPA_ERR_INVALID, "B, N, Hq, Hkv must be >= 1");
    if (Hq % Hkv) return fail(WPA_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (N >= (int64_t)INT32_MAX - wpa::kTileKeys) return fail(WPA_ERR_INVALID, "N too large");
    if (dtype != WPA_BF16) return fail(WPA_ERR_UNSUPPORTED, "the backward takes bf16 q, k, v and dout");
    if (out_dtype != WPA_BF16 && out_dtype != WPA_FP32) return fail(WPA_ERR_INVALID, "out_dtype must be WPA_BF16 or WPA_FP32");
    if (grad_dtype != WPA_BF16 && grad_dtype != WPA_FP32) return fail(WPA_ERR_INVALID, "grad_dtype must be WPA_BF16 or WPA_FP32");
    if (std::isnan(scale)) return fail(WPA_ERR_INVALID, "scale is NaN");
    if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !workspace)
        return fail(WPA_ERR_INVALID, "null pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace) ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return fail(WPA_ERR_INVALID, "tensors must be 16-byte aligned and the workspace 256-byte aligned");
    if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(WPA_ERR_INVALID, "lse must be 4-byte aligned");
    const BwdLayout L = bwd_layout(B, N, Hq, Hkv, d);
    if (ws_bytes < L.total) return fail(WPA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
    wpa::Tables tab;
    make_tables(d, base, rope, alpha, &tab);
    char* w = static_cast<char*>(workspace);
    wpa::BwdParams bp{};
    bp.q = q; bp.k = k; bp.v = v; bp.out = out; bp.lse = lse; bp.dout = dout;
    bp.dq = dq; bp.dk = dk; bp.dv = dv;
    bp.ks = reinterpret_cast<uint16_t*>(w + L.off[0]);
    bp.kt = reinterpret_cast<uint16_t*>(w + L.off[1]);
    bp.qs = reinterpret_cast<uint16_t*>(w + L.off[2]);
    bp.qt = reinterpret_cast<uint16_t*>(w + L.off[3]);
    bp.dot = reinterpret_cast<uint16_t*>(w + L.off[4]);
    bp.lse2 = reinterpret_cast<float*>(w + L.off[5]);
    bp.Dr = reinterpret_cast<float*>(w + L.off[6]);
    bp.dkp = reinterpret_cast<float*>(w + L.off[7]);
    bp.dvp = reinterpret_cast<float*>(w + L.off[8]);
    bp.vb = reinterpret_cast<uint16_t*>(w + L.off[9]);
    bp.dob = reinterpret_cast<uint16_t*>(w + L.off[10]);
    bp.N = N; bp.Np = round_up(N, wpa::kTileKeys);
    bp.B = B; bp.Hq = Hq; bp.Hkv = Hkv; bp.d = d;
    bp.out_f32 = out_dtype == WPA_FP32; bp.grad_f32 = grad_dtype == WPA_FP32;
    bp.interleaved = interleaved(rope);
    bp.scale = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)d));
    if (debug_on()) {
        const size_t nq = (size_t)B * N * Hq * d, nk = (size_t)B * N * Hkv * d, eg = esize(grad_dtype);
        if ((rc = dbg_extent(q, nq * 2, "q")) || (rc = dbg_extent(k, nk * 2, "k")) ||
            (rc = dbg_extent(v, nk * 2, "v")) || (rc = dbg_extent(out, nq * esize(out_dtype), "out")) ||
            (rc = dbg_extent(lse, (size_t)B * Hq * N * 4, "lse")) || (rc = dbg_extent(dout, nq * 2, "dout")) ||
            (rc = dbg_extent(dq, nq * eg, "dq")) || (rc = dbg_extent(dk, nk * eg, "dk")) ||
            (rc = dbg_extent(dv, nk * eg, "dv")) || (rc = dbg_extent(workspace, L.total, "workspace")))
            return rc;
    }
    hipError_t e = wpa::launch_backward(bp, tab, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(WPA_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
    if (debug_on()) return dbg_finish(stream, "prefill backward");
    return ok();
}

size_t wpa_kcache_bytes(int32_t B, int64_t Lmax, int32_t Hkv, int32_t d) {
    if (B < 1 || Lmax < 1 || Hkv < 1 || d < 1) return 0;
    return (size_t)B * Hkv * Lmax * d * 2;
}

size_t wpa_vcache_bytes(int32_t B, int64_t Lmax, int32_t Hkv, int32_t d) {
    if (B < 1 || Lmax < 1 || Hkv < 1 || d < 1) return 0;
    return (size_t)B * Hkv * ((Lmax + 7) / 8) * 8 * d * 2;
}

int wpa_kv_write(const void* k, const void* v, int64_t start, int64_t n, void* k_cache,
                 void* v_cache, int32_t B, int64_t Lmax, int32_t Hkv, int32_t d, double base,
                 int32_t dtype, void* stream) {
    return wpa_kv_write_ex(k, v, start, n, k_cache, v_cache, B, Lmax, Hkv, d, base, nullptr, dtype,
                           stream);
}

}  // extern "C"

namespace {

int kv_write_impl(const void* k, const void* v, int64_t start, int64_t n, void* k_cache,
                  void* v_cache, int32_t B, int64_t Lmax, int32_t Hkv, int32_t d, double base,
                  const wpa_rope_t* rope, const wpa::KLayout& kl, int32_t dtype, void* stream,
                  const wpa::Paging& pg = wpa::Paging{}) {
    if (B < 1 || Hkv < 1 || Lmax < 1 || n < 1 || start < 0 || start + n > Lmax)
        return fail(WPA_ERR_INVALID, "need B, Hkv, n >= 1 and 0 <= start, start + n <= Lmax");
    if (Lmax >= (int64_t)INT32_MAX) return fail(WPA_ERR_INVALID, "Lmax too large");
    if (dtype != WPA_BF16 && dtype != WPA_FP32) return fail(WPA_ERR_INVALID, "dtype must be WPA_BF16 or WPA_FP32");
    if (!k || !v || !k_cache || !v_cache) return fail(WPA_ERR_INVALID, "null pointer");
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(WPA_ERR_INVALID, "pointers must be 16-byte aligned");
    wpa::Tables tab;
    make_tables(d, base, rope, 1.0, &tab);
    wpa::RopeParams rp{};
    rp.interleaved = interleaved(rope);
    rp.k = k; rp.v = v; rp.pos = nullptr;
    rp.kp = static_cast<uint16_t*>(k_cache); rp.vout = static_cast<uint16_t*>(v_cache);
    rp.kl = kl;
    rp.n = n; rp.t0 = start; rp.ld = Lmax; rp.pad_to = 0;
    rp.B = B; rp.Hkv = Hkv; rp.d = d; rp.in_f32 = dtype == WPA_FP32; rp.v_prefill = 0;
    rp.tab = &tab;
    rp.pg = pg;
    rp.head_theta = head_tables(rope);
    if (debug_on()) {
        const size_t src = (size_t)B * n * Hkv * d * esize(dtype);
        int rc;
        if ((rc = dbg_extent(k, src, "k")) || (rc = dbg_extent(v, src, "v")) ||
            (rc = dbg_caches(k_cache, v_cache, B, Lmax, Hkv, d, kl, pg, std::vector<int64_t>(B, start),
                             std::vector<int64_t>(B, start + n), stream)) ||
            (rc = dbg_head_tables(rope, Hkv, d, stream)))
            return rc;
    }
    hipError_t e = wpa::launch_rope_relayout(rp, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(WPA_ERR_HIP, "kv write launch: %s", hipGetErrorString(e));
    if (debug_on()) return dbg_finish(stream, "kv write");
    return ok();
}

int decode_impl(const void* q, const void* k_cache, const void* v_cache, const int32_t* kv_len,
                const int32_t* q_pos, void* out, float* lse, int32_t B, int64_t Lmax,
                int32_t Hq, int32_t Hkv, int32_t d, double base, const wpa_rope_t* rope,
                const wpa::KLayout& kl, double alpha, float scale, int32_t dtype, int32_t out_dtype,
                unsigned long long* term_count, int32_t chunk_keys, void* workspace,
                size_t ws_bytes, void* stream, const wpa::Paging& pg = wpa::Paging{},
                bool use_scratch = false) {
    // use_scratch: the partials go to the library's per-GPU scratch array (workspace and
    // ws_bytes are ignored)
    if (B < 1 || Lmax < 1 || Hq < 1 || Hkv < 1) return fail(WPA_ERR_INVALID, "B, Lmax, Hq, Hkv must be >= 1");
    if (Hq % Hkv) return fail(WPA_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (Hq / Hkv > 16) return fail(WPA_ERR_UNSUPPORTED, "decode supports up to 16 q heads per kv head");
    if (Lmax >= (int64_t)INT32_MAX) return fail(WPA_ERR_INVALID, "Lmax too large");
    if (dtype != WPA_BF16 && dtype != WPA_FP32) return fail(WPA_ERR_INVALID, "dtype must be WPA_BF16 or WPA_FP32");
    if (out_dtype != WPA_BF16 && out_dtype != WPA_FP32) return fail(WPA_ERR_INVALID, "out_dtype must be WPA_BF16 or WPA_FP32");
    if (std::isnan(scale)) return fail(WPA_ERR_INVALID, "scale is NaN");
    if (chunk_keys < 0 || (chunk_keys % 256)) return fail(WPA_ERR_INVALID, "chunk_keys must be 0 or a positive multiple of 256");
    if (!q || !k_cache || !v_cache || !kv_len || !out || (!use_scratch && !workspace))
        return fail(WPA_ERR_INVALID, "null pointer");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        (!use_scratch && !aligned16(workspace)))
        return fail(WPA_ERR_INVALID, "q, caches, out and workspace must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(kv_len) & 3u) || (reinterpret_cast<uintptr_t>(q_pos) & 3u) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u))
        return fail(WPA_ERR_INVALID, "kv_len, q_pos and lse must be 4-byte aligned");
    if (term_count && (reinterpret_cast<uintptr_t>(term_count) & 7u)) return fail(WPA_ERR_INVALID, "term_count must be 8-byte aligned");
    const int ch = chunk_keys > 0 ? chunk_keys : default_chunk(B, Lmax, Hkv);
    const size_t need = wpa_decode_workspace_bytes(B, Lmax, Hq, Hkv, d, ch);
    if (use_scratch) {
        if (need > wpa::kDecodeScratchBytes)
            return fail(WPA_ERR_UNSUPPORTED, "decode partials need %zu bytes; the no-allocation entry point "
                        "holds %zu (use a larger chunk_keys, or wpa_decode_ex with a workspace)", need,
                        wpa::kDecodeScratchBytes);
        const hipError_t e = wpa::decode_scratch(&workspace);
        if (e != hipSuccess) return fail(WPA_ERR_HIP, "scratch address: %s", hipGetErrorString(e));
        ws_bytes = wpa::kDecodeScratchBytes;
    }
    if (ws_bytes < need) return fail(WPA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    wpa::Tables tab;
    make_tables(d, base, rope, alpha, &tab);
    wpa::DecodeParams dp{};
    dp.interleaved = interleaved(rope);
    dp.q = q; dp.kp = static_cast<const uint16_t*>(k_cache); dp.v = static_cast<const uint16_t*>(v_cache);
    dp.kl = kl;
    dp.kv_len = kv_len; dp.q_pos = q_pos; dp.out = out; dp.lse = lse; dp.counter = term_count;
    dp.partial = static_cast<float*>(workspace); dp.Lmax = Lmax; dp.B = B; dp.Hq = Hq; dp.Hkv = Hkv;
    dp.d = d; dp.in_f32 = dtype == WPA_FP32; dp.out_f32 = out_dtype == WPA_FP32; dp.chunk = ch; dp.n_chunks = (int)((Lmax + ch - 1) / ch);
    dp.balanced = chunk_keys == 0;
    dp.scale = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)d));
    dp.pg = pg;
    dp.head_theta = head_tables(rope);
    dp.alpha = alpha;
    if (debug_on()) {
        // (kv_len values are clamped by the kernels: not a precondition, but the pages the
        // clamped lengths reach must be in the pool)
        const size_t qo = (size_t)B * Hq * d;
        std::vector<int32_t> len;
        int rc;
        if ((rc = dbg_extent(q, qo * esize(dtype), "q")) || (rc = dbg_extent(out, qo * esize(out_dtype), "out")) ||
            (rc = dbg_extent(lse, (size_t)B * Hq * 4, "lse")) || (rc = dbg_extent(term_count, 8, "term_count")) ||
            (rc = dbg_extent(kv_len, (size_t)B * 4, "kv_len")) || (rc = dbg_extent(q_pos, (size_t)B * 4, "q_pos")) ||
            (!use_scratch && (rc = dbg_extent(workspace, need, "workspace"))) ||
            (rc = dbg_fetch(kv_len, (size_t)B, &len, stream, "kv_len")) ||
            (rc = dbg_head_tables(rope, Hkv, d, stream)))
            return rc;
        std::vector<int64_t> t1(B);
        for (int32_t b = 0; b < B; ++b) t1[b] = len[b] < 0 ? 0 : (len[b] > Lmax ? Lmax : len[b]);
        if ((rc = dbg_caches(k_cache, v_cache, B, Lmax, Hkv, d, kl, pg, std::vector<int64_t>(B, 0), t1,
                             stream)))
            return rc;
    }
    hipError_t e = wpa::launch_decode(dp, tab, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(WPA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    if (debug_on()) return dbg_finish(stream, "decode");
    return ok();
}

// Room of one key split of a cached prefill (outputs and log2-sums of every row and q head).
size_t split_bytes(int32_t B, int32_t Nq, int32_t Hq, int32_t d) {
    return (size_t)B * (size_t)Nq * (size_t)Hq * (size_t)(d + 1) * sizeof(float);
}

// cache_alpha of a windowed cache: finite (a full window keeps every key: use the dense
// cache), >= 0
int check_cache_alpha(double cache_alpha) {
    if (!(cache_alpha >= 0.0) || !std::isfinite(cache_alpha))
        return fail(WPA_ERR_INVALID, "cache_alpha must be finite and >= 0 (got %g)", cache_alpha);
    return WPA_OK;
}

int prefill_cached_impl(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* kv_len, void* out, float* lse, int32_t B, int32_t Nq,
                        int64_t Lmax, int32_t Hq, int32_t Hkv, int32_t d, double base,
                        const wpa_rope_t* rope, double alpha, float scale, int32_t dtype,
                        int32_t out_dtype, unsigned long long* term_count, void* stream,
                        const wpa::Paging& pg, const int32_t* cu_q, int32_t splits = 1,
                        void* workspace = nullptr, size_t ws_bytes = 0);

// A page table's description: page_size a power of two in [32, 65536] (a 32-token tile and
// an 8-token octet never straddle pages), the table's reach max_pages * page_size below 2^31.
int check_paging(const int32_t* table, int32_t num_pages, int32_t max_pages, int32_t page_size,
                 wpa::Paging* pg) {
    if (!table) return fail(WPA_ERR_INVALID, "null block table");
    if (num_pages < 1 || max_pages < 1) return fail(WPA_ERR_INVALID, "num_pages and max_pages must be >= 1");
    if (page_size < 32 || page_size > 65536 || (page_size & (page_size - 1)))
        return fail(WPA_ERR_INVALID, "page_size must be a power of two in [32, 65536] (got %d)", page_size);
    if ((int64_t)max_pages * page_size >= (int64_t)INT32_MAX)
        return fail(WPA_ERR_INVALID, "max_pages * page_size must be below 2^31");
    int lg = 0;
    while ((1 << lg) < page_size) ++lg;
    pg->table = table;
    pg->max_pages = max_pages;
    pg->page_log2 = lg;
    pg->num_pages = num_pages;
    return WPA_OK;
}

}  // namespace

extern "C" {

size_t wpa_kv_page_bytes(int32_t Hkv, int32_t d, int32_t page_size) {
    if (Hkv < 1 || (d != 64 && d != 128) || page_size < 32 || page_size > 65536 ||
        (page_size & (page_size - 1)))
        return 0;
    return (size_t)Hkv * d * page_size * 2;
}

int wpa_kv_write_paged(const void* k, const void* v, int64_t start, int64_t n, void* k_pool,
                       void* v_pool, const int32_t* block_table, int32_t num_pages, int32_t B,
                       int32_t max_pages, int32_t page_size, int32_t Hkv, int32_t d, double base,
                       const wpa_rope_t* rope, int32_t dtype, void* stream) {
    int rc = check_common(d, base, rope, 1.0);
    if (rc) return rc;
    wpa::Paging pg{};
    rc = check_paging(block_table, num_pages, max_pages, page_size, &pg);
    if (rc) return rc;
    return kv_write_impl(k, v, start, n, k_pool, v_pool, B, (int64_t)max_pages * page_size, Hkv,
                         d, base, rope, dense_layout(d, (int64_t)max_pages * page_size), dtype,
                         stream, pg);
}

int wpa_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_table, int32_t num_pages, const int32_t* kv_len,
                     const int32_t* q_pos, void* out, float* lse, int32_t B, int32_t max_pages,
                     int32_t page_size, int32_t Hq, int32_t Hkv, int32_t d, double base,
                     const wpa_rope_t* rope, double alpha, float scale, int32_t dtype,
                     int32_t out_dtype, unsigned long long* term_count, int32_t chunk_keys,
                     void* workspace, size_t ws_bytes, void* stream) {
    int rc = check_common(d, base, rope, alpha);
    if (rc) return rc;
    wpa::Paging pg{};
    rc = check_paging(block_table, num_pages, max_pages, page_size, &pg);
    if (rc) return rc;
    const int64_t Lmax = (int64_t)max_pages * page_size;
    return decode_impl(q, k_pool, v_pool, kv_len, q_pos, out, lse, B, Lmax, Hq, Hkv, d, base,
                       rope, dense_layout(d, Lmax), alpha, scale, dtype, out_dtype, term_count,
                       chunk_keys, workspace, ws_bytes, stream, pg);
}

int wpa_kv_write_ex(const void* k, const void* v, int64_t start, int64_t n, void* k_cache,
                    void* v_cache, int32_t B, int64_t Lmax, int32_t Hkv, int32_t d, double base,
                    const wpa_rope_t* rope, int32_t dtype, void* stream) {
    int rc = check_common(d, base, rope, 1.0);
    if (rc) return rc;
    return kv_write_impl(k, v, start, n, k_cache, v_cache, B, Lmax, Hkv, d, base, rope,
                         dense_layout(d, Lmax), dtype, stream);
}

size_t wpa_kcache_window_bytes(int32_t B, int64_t Lmax, int32_t Hkv, int32_t d, double base,
                               const wpa_rope_t* rope, double cache_alpha) {
    if (B < 1 || Lmax < 1 || Hkv < 1 || Lmax >= (int64_t)INT32_MAX) return 0;
    if (check_common(d, base, rope, 1.0) || check_cache_alpha(cache_alpha)) return 0;
    if (no_head_tables(rope, "a windowed cache")) return 0;
    return (size_t)B * Hkv * window_layout(d, Lmax, base, rope, cache_alpha).head * 32;
}

int wpa_kv_write_window(const void* k, const void* v, int64_t start, int64_t n, void* k_cache,
                        void* v_cache, int32_t B, int64_t Lmax, int32_t Hkv, int32_t d,
                        double base, const wpa_rope_t* rope, double cache_alpha, int32_t dtype,
                        void* stream) {
    int rc = check_common(d, base, rope, 1.0);
    if (rc) return rc;
    rc = check_cache_alpha(cache_alpha);
    if (rc) return rc;
    rc = no_head_tables(rope, "wpa_kv_write_window");
    if (rc) return rc;
    return kv_write_impl(k, v, start, n, k_cache, v_cache, B, Lmax, Hkv, d, base, rope,
                         window_layout(d, Lmax, base, rope, cache_alpha), dtype, stream);
}

int wpa_decode_window(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* kv_len, void* out, float* lse, int32_t B, int64_t Lmax,
                      int32_t Hq, int32_t Hkv, int32_t d, double base, const wpa_rope_t* rope,
                      double cache_alpha, double alpha, float scale, int32_t dtype,
                      int32_t out_dtype, unsigned long long* term_count, int32_t chunk_keys,
                      void* workspace, size_t ws_bytes, void* stream) {
    int rc = check_common(d, base, rope, alpha);
    if (rc) return rc;
    rc = check_cache_alpha(cache_alpha);
    if (rc) return rc;
    rc = no_head_tables(rope, "wpa_decode_window");
    if (rc) return rc;
    if (alpha > cache_alpha)
        return fail(WPA_ERR_INVALID, "alpha (%g) exceeds the cache's window alpha (%g)", alpha, cache_alpha);
    return decode_impl(q, k_cache, v_cache, kv_len, nullptr, out, lse, B, Lmax, Hq, Hkv, d, base,
                       rope, window_layout(d, Lmax, base, rope, cache_alpha), alpha, scale, dtype,
                       out_dtype, term_count, chunk_keys, workspace, ws_bytes, stream);
}

size_t wpa_decode_workspace_bytes(int32_t B, int64_t Lmax, int32_t Hq, int32_t Hkv, int32_t d,
                                  int32_t chunk_keys) {
    if (B < 1 || Lmax < 1 || Hq < 1 || Hkv < 1 || d < 1 || Hq % Hkv) return 0;
    const int ch = chunk_keys > 0 ? chunk_keys : default_chunk(B, Lmax, Hkv);
    const int64_t nc = (Lmax + ch - 1) / ch;
    return (size_t)B * Hkv * nc * (Hq / Hkv) * (d + 2) * sizeof(float);
}

int wpa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* kv_len,
               const int32_t* q_pos, void* out, float* lse, int32_t B, int64_t Lmax,
               int32_t Hq, int32_t Hkv, int32_t d, double base, double alpha, float scale,
               int32_t dtype, int32_t out_dtype, unsigned long long* term_count,
               int32_t chunk_keys, void* workspace, size_t ws_bytes, void* stream) {
    return wpa_decode_ex(q, k_cache, v_cache, kv_len, q_pos, out, lse, B, Lmax, Hq, Hkv, d, base,
                         nullptr, alpha, scale, dtype, out_dtype, term_count, chunk_keys, workspace,
                         ws_bytes, stream);
}

int wpa_decode_ex(const void* q, const void* k_cache, const void* v_cache, const int32_t* kv_len,
                  const int32_t* q_pos, void* out, float* lse, int32_t B, int64_t Lmax,
                  int32_t Hq, int32_t Hkv, int32_t d, double base, const wpa_rope_t* rope,
                  double alpha, float scale, int32_t dtype, int32_t out_dtype,
                  unsigned long long* term_count, int32_t chunk_keys, void* workspace,
                  size_t ws_bytes, void* stream) {
    int rc = check_common(d, base, rope, alpha);
    if (rc) return rc;
    return decode_impl(q, k_cache, v_cache, kv_len, q_pos, out, lse, B, Lmax, Hq, Hkv, d, base,
                       rope, dense_layout(d, Lmax), alpha, scale, dtype, out_dtype, term_count,
                       chunk_keys, workspace, ws_bytes, stream);
}

int wpa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* kv_len, const int32_t* q_pos, void* out, float* lse,
                       int32_t B, int64_t Lmax, int32_t Hq, int32_t Hkv, int32_t d, double base,
                       const wpa_rope_t* rope, double alpha, float scale, int32_t dtype,
                       int32_t out_dtype, unsigned long long* term_count, int32_t chunk_keys,
                       void* stream) {
    int rc = check_common(d, base, rope, alpha);
    if (rc) return rc;
    return decode_impl(q, k_cache, v_cache, kv_len, q_pos, out, lse, B, Lmax, Hq, Hkv, d, base,
                       rope, dense_layout(d, Lmax), alpha, scale, dtype, out_dtype, term_count,
                       chunk_keys, nullptr, 0, stream, wpa::Paging{}, true);
}

int wpa_prefill_cached(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* kv_len, void* out, float* lse, int32_t B, int32_t Nq,
                       int64_t Lmax, int32_t Hq, int32_t Hkv, int32_t d, double base,
                       const wpa_rope_t* rope, double alpha, float scale, int32_t dtype,
                       int32_t out_dtype, unsigned long long* term_count, void* stream) {
    return prefill_cached_impl(q, k_cache, v_cache, kv_len, out, lse, B, Nq, Lmax, Hq, Hkv, d,
                               base, rope, alpha, scale, dtype, out_dtype, term_count, stream,
                               wpa::Paging{}, nullptr);
}

int wpa_prefill_cached_varlen(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* cu_q, const int32_t* kv_len, void* out, float* lse,
                              int32_t B, int32_t max_q, int64_t Lmax, int32_t Hq, int32_t Hkv,
                              int32_t d, double base, const wpa_rope_t* rope, double alpha,
                              float scale, int32_t dtype, int32_t out_dtype,
                              unsigned long long* term_count, void* stream) {
    if (!cu_q || (reinterpret_cast<uintptr_t>(cu_q) & 3u)) return fail(WPA_ERR_INVALID, "cu_q must be a 4-byte aligned device pointer");
    return prefill_cached_impl(q, k_cache, v_cache, kv_len, out, lse, B, max_q, Lmax, Hq, Hkv, d,
                               base, rope, alpha, scale, dtype, out_dtype, term_count, stream,
                               wpa::Paging{}, cu_q);
}

int wpa_prefill_paged(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_table, int32_t num_pages, const int32_t* kv_len,
                      void* out, float* lse, int32_t B, int32_t Nq, int32_t max_pages,
                      int32_t page_size, int32_t Hq, int32_t Hkv, int32_t d, double base,
                      const wpa_rope_t* rope, double alpha, float scale, int32_t dtype,
                      int32_t out_dtype, unsigned long long* term_count, void* stream) {
    wpa::Paging pg{};
    int rc = check_paging(block_table, num_pages, max_pages, page_size, &pg);
    if (rc) return rc;
    return prefill_cached_impl(q, k_pool, v_pool, kv_len, out, lse, B, Nq,
                               (int64_t)max_pages * page_size, Hq, Hkv, d, base, rope, alpha,
                               scale, dtype, out_dtype, term_count, stream, pg, nullptr);
}

int wpa_prefill_paged_varlen(const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_table, int32_t num_pages, const int32_t* cu_q,
                             const int32_t* kv_len, void* out, float* lse, int32_t B,
                             int32_t max_q, int32_t max_pages, int32_t page_size, int32_t Hq,
                             int32_t Hkv, int32_t d, double base, const wpa_rope_t* rope,
                             double alpha, float scale, int32_t dtype, int32_t out_dtype,
                             unsigned long long* term_count, void* stream) {
    wpa::Paging pg{};
    int rc = check_paging(block_table, num_pages, max_pages, page_size, &pg);
    if (rc) return rc;
    if (!cu_q || (reinterpret_cast<uintptr_t>(cu_q) & 3u)) return fail(WPA_ERR_INVALID, "cu_q must be a 4-byte aligned device pointer");
    return prefill_cached_impl(q, k_pool, v_pool, kv_len, out, lse, B, max_q,
                               (int64_t)max_pages * page_size, Hq, Hkv, d, base, rope, alpha,
                               scale, dtype, out_dtype, term_count, stream, pg, cu_q);
}

size_t wpa_prefill_cached_workspace_bytes(int32_t B, int32_t Nq, int32_t Hq, int32_t Hkv,
                                          int32_t d, int32_t splits) {
    if (B < 1 || Nq < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || (d != 64 && d != 128) || splits < 0 ||
        splits > wpa::kMaxKeySplits || splits == 1)
        return 0;
    int ns = splits;
    if (ns == 0) {
        // the launch's own choice on the current device, with room for every split
        wpa::PrefillParams pp{};
        static const int32_t marker = 0;
        pp.kv_len = &marker;             // a cached launch (never read here)
        pp.part = reinterpret_cast<float*>(16);
        pp.max_splits = wpa::kMaxKeySplits;
        pp.Nq = Nq; pp.B = B; pp.Hq = Hq; pp.Hkv = Hkv; pp.d = d;
        ns = wpa::prefill_key_splits(pp);
    }
    return ns > 1 ? (size_t)ns * split_bytes(B, Nq, Hq, d) : 0;
}

int wpa_prefill_cached_ex(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, int32_t num_pages, int32_t page_size,
                          const int32_t* cu_q, const int32_t* kv_len, void* out, float* lse,
                          int32_t B, int32_t Nq, int64_t Lmax, int32_t Hq, int32_t Hkv, int32_t d,
                          double base, const wpa_rope_t* rope, double alpha, float scale,
                          int32_t dtype, int32_t out_dtype, unsigned long long* term_count,
                          int32_t splits, void* workspace, size_t ws_bytes, void* stream) {
    if (cu_q && (reinterpret_cast<uintptr_t>(cu_q) & 3u)) return fail(WPA_ERR_INVALID, "cu_q must be 4-byte aligned");
    wpa::Paging pg{};
    if (block_table) {
        if (page_size < 1 || Lmax % page_size || Lmax / page_size > INT32_MAX)
            return fail(WPA_ERR_INVALID, "Lmax (%lld) must be a multiple of page_size (%d)", (long long)Lmax, page_size);
        int rc = check_paging(block_table, num_pages, (int32_t)(Lmax / page_size), page_size, &pg);
        if (rc) return rc;
    }
    return prefill_cached_impl(q, k_cache, v_cache, kv_len, out, lse, B, Nq, Lmax, Hq, Hkv, d,
                               base, rope, alpha, scale, dtype, out_dtype, term_count, stream, pg,
                               cu_q, splits, workspace, ws_bytes);
}

}  // extern "C"

namespace {

int prefill_cached_impl(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* kv_len, void* out, float* lse, int32_t B, int32_t Nq,
                        int64_t Lmax, int32_t Hq, int32_t Hkv, int32_t d, double base,
                        const wpa_rope_t* rope, double alpha, float scale, int32_t dtype,
                        int32_t out_dtype, unsigned long long* term_count, void* stream,
                        const wpa::Paging& pg, const int32_t* cu_q, int32_t splits,
                        void* workspace, size_t ws_bytes) {
    int rc = check_common(d, base, rope, alpha);
    if (rc) return rc;
    if (B < 1 || Nq < 1 || Lmax < 1 || Hq < 1 || Hkv < 1) return fail(WPA_ERR_INVALID, "B, Nq, Lmax, Hq, Hkv must be >= 1");
    if (Nq > Lmax) return fail(WPA_ERR_INVALID, "Nq (%d) exceeds Lmax (%lld)", Nq, (long long)Lmax);
    if (Hq % Hkv) return fail(WPA_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (Lmax >= (int64_t)INT32_MAX - 64) return fail(WPA_ERR_INVALID, "Lmax too large");
    if (dtype != WPA_BF16 && dtype != WPA_FP32) return fail(WPA_ERR_INVALID, "dtype must be WPA_BF16 or WPA_FP32");
    if (out_dtype != WPA_BF16 && out_dtype != WPA_FP32) return fail(WPA_ERR_INVALID, "out_dtype must be WPA_BF16 or WPA_FP32");
    if (std::isnan(scale)) return fail(WPA_ERR_INVALID, "scale is NaN");
    if (!q || !k_cache || !v_cache || !kv_len || !out) return fail(WPA_ERR_INVALID, "null pointer");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return fail(WPA_ERR_INVALID, "q, caches and out must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(kv_len) & 3u) return fail(WPA_ERR_INVALID, "kv_len must be 4-byte aligned");
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(WPA_ERR_INVALID, "lse must be 4-byte aligned");
    if (term_count && (reinterpret_cast<uintptr_t>(term_count) & 7u)) return fail(WPA_ERR_INVALID, "term_count must be 8-byte aligned");
    wpa::Tables tab;
    make_tables(d, base, rope, alpha, &tab);
    wpa::PrefillParams pp{};
    pp.interleaved = interleaved(rope);
    pp.q = q; pp.kp = static_cast<const uint16_t*>(k_cache); pp.vt = static_cast<const uint16_t*>(v_cache);
    pp.kv_len = kv_len; pp.out = out; pp.lse = lse; pp.pos = nullptr; pp.counter = term_count;
    pp.N = Lmax; pp.Np = 0; pp.ldk = Lmax; pp.Nq = Nq; pp.B = B; pp.Hq = Hq;
    pp.Hkv = Hkv; pp.d = d; pp.in_f32 = dtype == WPA_FP32; pp.out_f32 = out_dtype == WPA_FP32;
    pp.scale = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)d));
    pp.pg = pg;
    pp.cu_q = cu_q;
    pp.head_theta = head_tables(rope);
    pp.alpha = alpha;                  // (per-head tables: windows computed on the device)
    if (splits < 0 || splits > wpa::kMaxKeySplits)
        return fail(WPA_ERR_INVALID, "splits must be in [0, %d] (got %d)", wpa::kMaxKeySplits, splits);
    if (splits != 1 && workspace) {
        if (!aligned16(workspace)) return fail(WPA_ERR_INVALID, "workspace must be 16-byte aligned");
        // the splits the workspace has room for
        const size_t per = split_bytes(B, Nq, Hq, d);
        const size_t fit = ws_bytes / per;
        pp.part = static_cast<float*>(workspace);
        pp.max_splits = (int32_t)(fit < (size_t)wpa::kMaxKeySplits ? fit : (size_t)wpa::kMaxKeySplits);
        pp.splits = splits;
        if (splits > 1 && pp.max_splits < splits)
            return fail(WPA_ERR_INVALID, "workspace of %zu bytes holds %d key splits, %d asked for",
                        ws_bytes, pp.max_splits, splits);
    } else if (splits > 1) {
        return fail(WPA_ERR_INVALID, "%d key splits need a workspace", splits);
    }
    if (debug_on()) {
        // kv_len[b] in [q_b, Lmax]; cu_q non-decreasing from >= 0 with q_b <= Nq
        std::vector<int32_t> len, cu;
        if ((rc = dbg_extent(kv_len, (size_t)B * 4, "kv_len")) ||
            (rc = dbg_extent(cu_q, (size_t)(B + 1) * 4, "cu_q")) ||
            (rc = dbg_fetch(kv_len, (size_t)B, &len, stream, "kv_len")) ||
            (rc = dbg_fetch(cu_q, cu_q ? (size_t)B + 1 : 0, &cu, stream, "cu_q")) ||
            (rc = dbg_head_tables(rope, Hkv, d, stream)))
            return rc;
        if (cu_q && cu[0] < 0) return fail(WPA_ERR_INVALID, "debug: cu_q[0] = %d is negative", cu[0]);
        std::vector<int64_t> t1(B);
        for (int32_t b = 0; b < B; ++b) {
            const int64_t qb = cu_q ? (int64_t)cu[b + 1] - cu[b] : Nq;
            if (qb < 0 || qb > Nq)
                return fail(WPA_ERR_INVALID, "debug: sequence %d has %lld queries (allowed 0 .. %d)", b,
                            (long long)qb, Nq);
            if (len[b] < qb || len[b] > Lmax)
                return fail(WPA_ERR_INVALID, "debug: kv_len[%d] = %d is outside [%lld, %lld]", b, len[b],
                            (long long)qb, (long long)Lmax);
            t1[b] = len[b];
        }
        const size_t rows = cu_q ? (size_t)cu[B] : (size_t)B * Nq;
        if ((rc = dbg_extent(q, rows * Hq * d * esize(dtype), "q")) ||
            (rc = dbg_extent(out, rows * Hq * d * esize(out_dtype), "out")) ||
            (rc = dbg_extent(lse, rows * Hq * 4, "lse")) || (rc = dbg_extent(term_count, 8, "term_count")) ||
            (rc = dbg_extent(pp.part ? workspace : nullptr, ws_bytes, "workspace")) ||
            (rc = dbg_caches(k_cache, v_cache, B, Lmax, Hkv, d, dense_layout(d, Lmax), pg,
                             std::vector<int64_t>(B, 0), t1, stream)))
            return rc;
    }
    hipError_t e = wpa::launch_prefill(pp, tab, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(WPA_ERR_HIP, "cached prefill launch: %s", hipGetErrorString(e));
    if (debug_on()) return dbg_finish(stream, "cached prefill");
    return ok();
}

}  // namespace

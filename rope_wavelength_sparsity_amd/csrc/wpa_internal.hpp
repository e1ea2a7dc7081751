// Internal launch interface between the C-ABI layer (wpa_api.cpp) and the HIP kernels.
// Host-visible plain structs only; no HIP types beyond hipStream_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wpa {

constexpr int kMaxPairs = 64;     // d <= 128
constexpr int kTileKeys = 128;    // token padding of the prefill workspace (a multiple of every key tile)

// Window and rotation tables, computed once on the host in double.
struct Tables {
    int32_t W[kMaxPairs];         // floor(alpha*lambda_i), INT32_MAX when unbounded
    double theta[kMaxPairs];      // rotation frequency of pair i (base^(-2i/d), or a table)
};

// Rotate keys into the pair-blocked layout [B][Hkv][d/16][ld][16] (IEEE half) and write V
// by key octets, [B][Hkv][ceil(ld/8)][d][8] (bf16), for the prefill workspace and the decode
// cache alike.  Tokens t0 .. t0+n-1 of the destination receive source rows 0 .. n-1; tokens
// n .. pad_to-1 (prefill only) are zero-filled.
// Rows of the pair-blocked K layout of one (sequence, kv head): block j holds cap[j] rows
// starting at row off[j].  A block with fewer rows than the tokens it serves is a ring:
// token t sits in row t mod cap[j] (cap[j] a multiple of 32, so a 32-token tile starting at a
// multiple of 32 never wraps).  Dense layouts have cap[j] = tokens, off[j] = j * tokens.
struct KLayout {
    int64_t head;                 // rows per (sequence, kv head)
    int64_t off[8];
    int32_t cap[8];
};

// Paged caches: the token range [i*page, (i+1)*page) of sequence b lives in page
// table[b*max_pages + i] of a pool.  A K page is [Hkv][d/16][page][16] half (pair-blocked),
// a V page [Hkv][page/8][d][8] bf16 (key octets); page is a power of two >= 32, so a 32-token
// tile and an octet never straddle pages.  table == null: contiguous per-sequence caches.
struct Paging {
    const int32_t* table;         // [B][max_pages] device, or null
    int32_t max_pages, page_log2, num_pages;
};

// Pool page holding token tok of sequence b (tok < max_pages << page_log2).  Entries outside
// [0, num_pages) break the caller's contract; they are clamped so that no access leaves the pool.
__device__ inline int64_t page_of(const Paging& pg, int b, int64_t tok) {
    const int64_t page = pg.table[(int64_t)b * pg.max_pages + (tok >> pg.page_log2)];
    return page < 0 ? 0 : (page >= pg.num_pages ? pg.num_pages - 1 : page);
}

struct RopeParams {
    const void* k;                // [B][n][Hkv][d]
    const void* v;                // [B][n][Hkv][d]
    const int32_t* pos;           // [B][n] or null (positions t0 + row)
    uint16_t* kp;                 // pair-blocked rotated keys, rows as in kl
    uint16_t* vout;               // values by key octets [B][Hkv][ld/8][d][8]
    KLayout kl;
    int64_t n, t0, ld, pad_to;
    int32_t B, Hkv, d, in_f32;
    int32_t v_prefill;            // the prefill workspace (all of it written, zero past n)
                                  // rather than a cache write (other tokens kept)
    int32_t interleaved;          // pair i = dims (2i, 2i+1) instead of (i, i+d/2)
    const Tables* tab;            // host pointer; copied into kernel arguments
    Paging pg;                    // decode cache writes: pages (table null: kl layout)
    const double* head_theta;     // [Hkv][d/2] device: per-kv-head frequencies, or null (tab)
};

struct PrefillParams {
    const void* q;                // [B][N][Hq][d]  (cached: [B][Nq][Hq][d])
    const uint16_t* kp;           // [B][Hkv][d/16][ldk][16]
    const uint16_t* vt;           // V by key octets [B][Hkv][Np/8][d][8]  (cached: the V cache
                                  // [B][Hkv][ceil(ldk/8)][d][8])
    const int32_t* kv_len;        // cached (chunked) prefill: [B] keys per sequence; else null
    int64_t ldk;                  // key row stride of kp: Np, or Lmax of the caches
    int32_t Nq;                   // cached: queries per sequence (its last Nq tokens)
    const int32_t* blk_count;     // block-sparse: [B][Hq][ceil(N/blk)] list lengths; else null
    const int32_t* blk_idx;       // block-sparse: [B][Hq][ceil(N/blk)][blk_max] key blocks
    int32_t blk_max;
    int32_t blk_log2;             // block-sparse: log2 of the block size blk (6 .. 10)
    void* out;                    // [B][N][Hq][d]
    float* lse;                   // [B][Hq][N] or null
    const int32_t* pos;           // [B][N] or null
    unsigned long long* counter;  // or null
    int64_t N, Np;                // N: tokens (cached: Lmax); Np: workspace padding
    int32_t B, Hq, Hkv, d, in_f32, out_f32;
    int32_t interleaved;          // pair i = dims (2i, 2i+1) instead of (i, i+d/2)
    float scale;
    Paging pg;                    // cached prefill on paged caches (kp, vt: the pools)
    const int32_t* cu_q;          // cached prefill, varlen: [B+1] first packed q row of each
                                  // sequence (q, out [rows][Hq][d], lse [rows][Hq]); else null
    const double* head_theta;     // [Hkv][d/2] device: per-kv-head frequencies (windows are
    double alpha;                 // computed from them and alpha in the kernel), or null (tab)
    // cached prefill: key splits (the row blocks' key tiles shared among up to max_splits
    // workgroups, their partials merged by a combine kernel) when part is set and
    // max_splits > 1; splits > 0 asks for exactly that many (capped), 0 lets the launch choose
    float* part;                  // [ns][B*Nq][Hq][d] outputs, then [ns][B*Nq][Hq] log2-sums
    int32_t max_splits, splits;
};

// Most key splits of one cached prefill launch.
constexpr int kMaxKeySplits = 16;

struct DecodeParams {
    const void* q;                // [B][Hq][d]
    const uint16_t* kp;           // [B][Hkv][rows as in kl][16]
    const uint16_t* v;            // [B][Hkv][ceil(Lmax/8)][d][8]
    KLayout kl;
    const int32_t* kv_len;        // [B]
    const int32_t* q_pos;         // [B] or null
    void* out;                    // [B][Hq][d]
    float* lse;                   // [B][Hq] or null
    unsigned long long* counter;
    float* partial;               // [B][Hkv][n_chunks][G][d+2]
    int64_t Lmax;
    int32_t B, Hq, Hkv, d, in_f32, out_f32, chunk, n_chunks;
    int32_t balanced;             // 1: chunks of equal streamed bytes, counted from the last key
                                  // (n_chunks of them); 0: chunk c = keys [c*chunk, (c+1)*chunk)
    int32_t interleaved;          // pair i = dims (2i, 2i+1) instead of (i, i+d/2)
    float scale;
    Paging pg;                    // pools of pages (table null: kl layout, [B][Hkv][..] V)
    const double* head_theta;     // [Hkv][d/2] device: per-kv-head frequencies, or null (tab)
    double alpha;
};

// Backward of the one-shot prefill (positions = token indices).  Inputs q, k, v, dout bf16
// ([B][N][H][d]), out (forward output, out_f32 ? fp32 : bf16), lse [B][Hq][N] fp32; outputs
// dq, dk, dv (grad_f32 ? fp32 : bf16) in the inputs' layouts.  Workspace regions (device):
struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* out;
    const float* lse;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    uint16_t* ks;                 // rotated K' pair-blocked [B][Hkv][d/16][Np][16] half
    uint16_t* kt;                 // rotated K'^T by key octets [B][Hkv][Np/8][d][8] half (pair-block
                                  // element order within a key's d)
    uint16_t* vb;                 // V blocked by 16 dims [B][Hkv][d/16][Np][16] bf16
    uint16_t* qs;                 // rotated Q' * scale*log2 e, pair-blocked [B][Hq][d/16][Np][16]
    uint16_t* qt;                 // rotated Q'^T (unscaled) by row octets [B][Hq][Np/8][d][8] half
    uint16_t* dot;                // dout^T by row octets [B][Hq][Np/8][d][8] bf16
    uint16_t* dob;                // dout blocked by 16 dims [B][Hq][d/16][Np][16] bf16
    float* lse2;                  // lse * log2 e [B][Hq][Np] (+inf past N)
    float* Dr;                    // dout . out [B][Hq][Np]
    float* dkp;                   // per-q-head dk'^T partials [B][Hq][Np][d] (pair-block order)
    float* dvp;                   // per-q-head dv partials [B][Hq][Np][d]
    int64_t N, Np;
    int32_t B, Hq, Hkv, d, out_f32, grad_f32;
    int32_t interleaved;
    float scale;
};

hipError_t launch_rope_relayout(const RopeParams& p, hipStream_t s);
hipError_t launch_backward(const BwdParams& p, const Tables& t, hipStream_t s);
hipError_t launch_prefill(const PrefillParams& p, const Tables& t, hipStream_t s);
// Key splits a cached prefill launch with these shapes would take on the current device
// (p.max_splits, p.splits as for the launch; 1: none).
int prefill_key_splits(const PrefillParams& p);
// LDS bytes a block-sparse prefill launch for p (d, dtype, N, counter) needs, and the
// device's per-workgroup limit; nothing is enqueued.
hipError_t prefill_sparse_lds(const PrefillParams& p, size_t* need, size_t* limit);
hipError_t launch_decode(const DecodeParams& p, const Tables& t, hipStream_t s);

// Size of the per-GPU scratch array of the no-allocation decode entry point (its split-KV
// partials), and its device address on the current device (looked up once per device).
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
hipError_t decode_scratch(void** ptr);

}  // namespace wpa

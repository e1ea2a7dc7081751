// One decode step with the per-RoPE-wavelength window (ATFlash abstract: the window
// ported into a decode kernel), split over the KV sequence, on MFMA (q.k in half
// precision, P*V in bf16).
//
// Work item = (sequence b, kv head g, chunk of `chunk` keys); items past kv_len exit.
// Each item serves all G q heads of its kv head, so every K/V byte is read once per step.
// The 4 waves take interleaved 32-key tiles of the chunk, each with its own online-softmax
// state, merged in LDS at the end.  A wave's next tile is in flight while it computes the
// current one.
//
// Per 32-key tile (one 32x32x16 MFMA row block):
//   S^T[32 keys x 32 cols] = K'[keys x 16 dims] * Q'^T, one MFMA per active 16-dim pair
//   block; columns are the G q heads (padded to 32).  With a single query position the
//   window test depends on the key alone, so straddling pairs are handled exactly by
//   zeroing them in the key's A-operand row (lane = key): no per-element fixup.  Blocks
//   below the first pair active anywhere in the tile are neither read nor multiplied: far
//   keys stream only the blocks of the long-wavelength pairs still inside their window.
//   Softmax runs per column (lane = q head) over the keys held in registers, exp2 domain
//   (q' is pre-scaled by scale*log2 e), lazy rescale.  The key rows of the A operand are
//   permuted (bits 2 and 3 swapped) so the S^T registers are directly the P^T operand of
//   O^T[32 dims x 32 cols] += V^T[32 dims x 16 keys] * P^T, whose V^T operand is one
//   16-byte load per lane from the key-octet-blocked V cache.
#include <atomic>

#include "wpa_device.hpp"
#include "wpa_internal.hpp"

namespace wpa {

// The no-allocation decode entry point keeps its split-KV partials here instead of in a
// caller workspace: one copy of this array per GPU, held until the process ends.  Host code
// must not use the array's name as an address (on the host it is only a stand-in); the
// device address comes from hipGetSymbolAddress, once per device (decode_scratch below).
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

namespace {

constexpr int kWaves = 4;
constexpr float kTau = 8.0f;
constexpr int kBufWord3 = 0x00020000;   // buffer descriptor word 3 (raw bytes, no format)
constexpr int kNT = 2;                  // buffer load cache policy: non-temporal

__device__ inline int perm_row(int m) {
    return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// A sequence's key count as the kernels use it: kv_len clamped into [0, Lmax].
__device__ inline int clamp_len(int32_t len, int64_t Lmax) {
    const int l = __builtin_amdgcn_readfirstlane(len);
    return l < 0 ? 0 : (l > Lmax ? (int)Lmax : l);
}

__device__ inline float xchg32(float v, int xaddr) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(xaddr, __builtin_bit_cast(int, v)));
}

// Byte-balanced split of a sequence's keys (the library's default).  A key at distance x
// from the sequence's last key streams its V row (2d bytes) and the K blocks still active at
// that distance, block j while x <= Wb[j], the window of its last pair (32 bytes each).  In
// units of 32 bytes the keys at distances below x stream
//     F(x) = x*d/16 + sum_j min(x, Wb[j] + 1),
// non-decreasing with slope in [d/16, d/8].  Over the span S = n*chunk of the launch's n chunks,
// chunk c takes the distances [dl_c, dl_{c+1}), dl_c the smallest x with F(x)*n >= c*F(S), i.e.
// chunks of equal bytes, and as keys the range [K_{c+1}, K_c) with K_0 = L and K_c = max(0,
// (L - dl_c) rounded down to 32) (tiles start on 32-key boundaries, as ring caches and pages
// need).  The split depends only on the window table and (n, chunk), so caches of different
// Lmax with the same chunk grid split alike.  Every chunk spans more than chunk/2 - 1 >= 127
// distances, so the non-empty chunks of a sequence of L keys are the first
// 1 + #{c >= 1 : dl_c <= L - 32}.
template <int NB>
struct ByteSplit {
    int64_t wb[NB];
    int64_t Ftot, n, S;
    int D;
    __device__ int64_t F(int64_t x) const {
        int64_t f = x * (D / 16);
#pragma unroll
        for (int j = 0; j < NB; ++j) f += x < wb[j] + 1 ? x : wb[j] + 1;
        return f;
    }
    // dl_c for c in [1, n): the smallest x in [0, S] with F(x)*n >= c*Ftot, i.e. F(x) >= T =
    // ceil(c*Ftot / n), found by walking F's linear pieces: on [Wb[j-1]+1, Wb[j]+1) the slope is
    // d/16 plus the blocks still active (Wb is non-decreasing in j).  (A binary search gave the
    // same bounds at ~20x the scalar instructions, which short decode steps felt.)
    __device__ int64_t bound(int64_t c) const {
        const int64_t T = (c * Ftot + n - 1) / n;
        int64_t x0 = 0, F0 = 0, slope = D / 16 + NB;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int64_t x1 = wb[j] + 1 < S ? wb[j] + 1 : S;
            if (x1 > x0) {
                if (F0 + slope * (x1 - x0) >= T) return x0 + (T - F0 > 0 ? (T - F0 + slope - 1) / slope : 0);
                F0 += slope * (x1 - x0);
                x0 = x1;
            }
            slope -= 1;
            if (x0 >= S) return S;
        }
        const int64_t x = x0 + (T - F0 > 0 ? (T - F0 + slope - 1) / slope : 0);
        return x < S ? x : S;
    }
    // K_c of a sequence of L keys (c in [0, n])
    __device__ int64_t key_bound(int64_t c, int64_t L) const {
        if (c == 0) return L;
        if (c >= n) return 0;
        const int64_t k = (L - bound(c)) & ~(int64_t)31;
        return k > 0 ? k : 0;
    }
    // number of non-empty chunks of a sequence of L keys
    __device__ int chunks_used(int64_t L) const {
        if (L <= 0) return 0;
        if (L < 32) return 1;
        const int64_t k = F(L - 32) * n / Ftot;       // #{c >= 1 : dl_c <= L - 32}, before the cap
        return 1 + (int)(k < n - 1 ? k : n - 1);
    }
};

// The split of kv head g: Wb[j] from the shared table or kv head g's frequencies.
template <int D>
__device__ inline ByteSplit<D / 16> byte_split(const DecodeParams& p, const Tables& tab, int g) {
    constexpr int NB = D / 16, P = D / 2;
    ByteSplit<NB> s;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int w = p.head_theta ? window_from_theta(p.alpha, p.head_theta[(int64_t)g * P + 8 * j + 7])
                                   : tab.W[8 * j + 7];
        s.wb[j] = w;
    }
    s.D = D;
    s.n = p.n_chunks;
    s.S = (int64_t)p.n_chunks * p.chunk;
    s.Ftot = s.F(s.S);
    return s;
}

template <int D, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void decode_partial_kernel(DecodeParams p, Tables tab) {
    constexpr int NB = D / 16;
    constexpr int P = D / 2;
    constexpr int NDB = D / 32;
    constexpr int GMAX = 16;                        // q heads per kv head (columns used)
    __shared__ __attribute__((aligned(16))) uint16_t sQ[32][D];      // pair-blocked, half
    __shared__ float sO[kWaves][GMAX][D + 2];

    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, h = lane >> 5;
    const int xaddr = (lane ^ 32) << 2;
    const int G = p.Hq / p.Hkv;
    const int chunk = blockIdx.x % p.n_chunks;
    const int bg = blockIdx.x / p.n_chunks;
    const int g = bg % p.Hkv, b = bg / p.Hkv;
    // kv_len is clamped into [0, Lmax] (the caches' or the block table's reach), so no access
    // leaves the caches whatever the device holds; a sequence with no keys writes no partial
    const int Lb = clamp_len(p.kv_len[b], p.Lmax);
    int key_lo, key_hi;
    if (p.balanced) {
        const ByteSplit<NB> bs = byte_split<D>(p, tab, g);
        key_hi = __builtin_amdgcn_readfirstlane((int)bs.key_bound(chunk, Lb));
        key_lo = __builtin_amdgcn_readfirstlane((int)bs.key_bound(chunk + 1, Lb));
    } else {
        key_lo = chunk * p.chunk;
        key_hi = key_lo + p.chunk < Lb ? key_lo + p.chunk : Lb;
    }
    if (key_lo >= key_hi) return;
    const int64_t qpos = __builtin_amdgcn_readfirstlane(p.q_pos ? p.q_pos[b] : Lb - 1);
    const float sl2 = p.scale * 1.4426950408889634f;
    uint64_t cnt = 0;

    // rotated q of the G heads (pre-scaled into log2 units), pair-blocked half-precision
    // rows; rows >= G are zero
    for (int i = tid; i < 32 * P; i += blockDim.x) {
        const int hh = i / P, pr = i % P;
        const int j = pr >> 3, e = pr & 7;
        float xo = 0.f, yo = 0.f;
        if (hh < G) {
            const int64_t qb = ((int64_t)b * p.Hq + g * G + hh) * D;
            // the two dims of pair pr: (pr, pr+P) half-split, (2pr, 2pr+1) interleaved
            const int64_t ix = p.interleaved ? qb + 2 * pr : qb + pr;
            const int64_t iy = p.interleaved ? ix + 1 : ix + P;
            float x, y;
            if (p.in_f32) {
                x = round_bf16(static_cast<const float*>(p.q)[ix]);
                y = round_bf16(static_cast<const float*>(p.q)[iy]);
            } else {
                x = bf16_bits_to_f32(static_cast<const uint16_t*>(p.q)[ix]);
                y = bf16_bits_to_f32(static_cast<const uint16_t*>(p.q)[iy]);
            }
            float sn, cs;
            rope_sincos(qpos, p.head_theta ? p.head_theta[(int64_t)g * P + pr] : tab.theta[pr], &sn, &cs);
            xo = (x * cs - y * sn) * sl2;
            yo = (y * cs + x * sn) * sl2;
        }
        sQ[hh][16 * j + e] = f32_to_f16_bits(xo);
        sQ[hh][16 * j + 8 + e] = f32_to_f16_bits(yo);
    }
    __syncthreads();
    // B operand of QK: column l32 = q head, half h = first/second halves of the block's pairs
    u32x4 qB[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) qB[j] = *reinterpret_cast<const u32x4*>(&sQ[l32][16 * j + 8 * h]);

    // (paged: the pools; a tile's page is looked up per tile)
    const uint16_t* kpg = PAGED ? p.kp : p.kp + ((int64_t)b * p.Hkv + g) * p.kl.head * 16;
    const int64_t L8 = (p.Lmax + 7) / 8;
    const uint16_t* vg = PAGED ? p.v : p.v + ((int64_t)b * p.Hkv + g) * L8 * D * 8;

    f32x16 O[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) O[i] = f32x16{};
    float m = -INFINITY, lsum = 0.f;
    const int arow = perm_row(l32);                  // key row this lane feeds to the A operand

    const char* kbytes = reinterpret_cast<const char*>(kpg);
    const char* vbytes = reinterpret_cast<const char*>(vg);
    const int koffl = arow * 32 + 16 * h;            // lane offset in a K block's 32 rows
    // window of pair `lane` (per-head tables: from kv head g's frequency)
    const int Wl = lane >= P ? INT32_MAX
                 : (p.head_theta ? window_from_theta(p.alpha, p.head_theta[(int64_t)g * P + lane])
                                 : tab.W[lane]);
    const int voffl = (h * D + l32) * 16;            // lane offset in a tile's V octets
    int plo = 0, pfull = 0;                          // band edges of the current tile

    // Band of the tile at k0: the first pair with W >= its smallest distance (plo) and
    // with W >= its largest (pfull), i.e. the numbers of pairs with W below them (W is
    // non-decreasing in the pair index): one ballot over the lane-held table each.
    auto band = [&](int k0) {
        const int kmax = k0 + 31 < key_hi ? k0 + 31 : key_hi - 1;
        int64_t dlo, dhi;
        if (qpos >= kmax) { dlo = qpos - kmax; dhi = qpos - k0; }
        else if (qpos <= k0) { dlo = k0 - qpos; dhi = kmax - qpos; }
        else { dlo = 0; dhi = (qpos - k0 > kmax - qpos) ? qpos - k0 : kmax - qpos; }
        const int dl = __builtin_amdgcn_readfirstlane((int)(dlo < INT32_MAX ? dlo : INT32_MAX));
        const int dh = __builtin_amdgcn_readfirstlane((int)(dhi < INT32_MAX ? dhi : INT32_MAX));
        plo = __builtin_popcountll(__ballot(Wl < dl));
        pfull = __builtin_popcountll(__ballot(Wl < dh));
    };
    // Loads of the tile at k0 (band already moved there) through buffer descriptors
    // whose extent holds only what is wanted: the K blocks below the band's first
    // active one, the rows past the chunk's last key and a whole tile past the chunk
    // get extent 0 and read as zero without touching memory.  So every tile issues the
    // same loads, and those of the next tile can be in flight while this one computes.
    // The caches are streamed once per step: non-temporal loads (a plain read runs
    // markedly closer to the HBM peak with them).
    // page of the tile at k0 (paged caches; 0 past the chunk, where nothing is read)
    auto tile_page = [&](int k0) -> int64_t {
        if constexpr (PAGED) return k0 < key_hi ? page_of(p.pg, b, k0) : 0;
        else return 0;
    };
    auto kload = [&](int k0, int64_t page, u32x4 (&ka)[NB]) {
        const int jlo = plo >> 3;
        const int nk = k0 < key_hi ? (key_hi - k0 < 32 ? key_hi - k0 : 32) : 0;
        if constexpr (PAGED) {
            // rows k0 mod page .. +31 of block j of (page, kv head g)
            const int ps = 1 << p.pg.page_log2;
            const int64_t row0 = (page * p.Hkv + g) * NB * ps + (k0 & (ps - 1));
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const char* base = kbytes + (row0 + (int64_t)j * ps) * 32;
                const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<char*>(base), 0, j >= jlo ? nk * 32 : 0, kBufWord3);
                ka[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, koffl, 0, kNT));
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            // rows of this tile in block j: from the key itself, or in a ring block (one
            // holding only the keys inside its largest window) from k0 mod cap; a tile
            // never wraps (cap is a multiple of 32)
            const int cap = p.kl.cap[j];
            const int r0 = cap < p.Lmax ? (int)((uint32_t)k0 % (uint32_t)cap) : k0;
            const char* base = kbytes + (p.kl.off[j] + r0) * 32;
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<char*>(base), 0, j >= jlo ? nk * 32 : 0, kBufWord3);
            ka[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, koffl, 0, kNT));
        }
    };
    // V^T operands of the tile at k0: lane = dim, half h = key octet; the octets past the
    // cache's end read as zero
    auto vload = [&](int k0, int64_t page, u32x4 (&va)[2][NDB]) {
        int64_t oct0 = k0 >> 3, nob = k0 < key_hi ? (L8 - oct0 < 4 ? L8 - oct0 : 4) : 0;
        if constexpr (PAGED) {
            // octet (k0 mod page)/8 of (page, kv head g); a tile never leaves its page
            const int o_pg = 1 << (p.pg.page_log2 - 3);
            oct0 = (page * p.Hkv + g) * o_pg + ((k0 >> 3) & (o_pg - 1));
            nob = k0 < key_hi ? 4 : 0;
        }
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(vbytes + oct0 * (D * 16)), 0, (int)nob * D * 16, kBufWord3);
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                va[c][db] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    rs, voffl + (2 * c * D + 32 * db) * 16, 0, kNT));
    };

    int k0 = key_lo + 32 * w;
    band(k0);
    u32x4 ka[NB], va[2][NDB];
    int64_t page = tile_page(k0);
    kload(k0, page, ka);
    vload(k0, page, va);
    while (k0 < key_hi) {
        const int pl = plo, pf = pfull, jlo = pl >> 3;   // this tile's band
        const bool tail = k0 + 32 > key_hi;          // tile runs past the chunk's last key
        const int key = k0 + arow;

        // S^T over the active blocks; pairs not active for this lane's key are zeroed.
        // Pairs below pl are dead and pairs from pf on active for every key of the tile;
        // the key's first active pair fa counts the straddling pairs whose window it
        // leaves (windows grow with the pair index).
        const int64_t dist = qpos - key >= 0 ? qpos - key : key - qpos;
        int fa = pl;
        for (int e = pl; e < pf; ++e) fa += dist > (int64_t)__builtin_amdgcn_readlane(Wl, e) ? 1 : 0;
        if (p.counter && h == 0 && key < key_hi) cnt += P - fa;
        f32x16 S = f32x16{};
#pragma unroll
        for (int j = NB - 1; j >= 0; --j) {
            if (j < jlo) continue;
            u32x4 a = ka[j];
            if (8 * j < pf) {                         // block holds a straddling pair
                const int lead = fa - 8 * j;          // its pairs below fa are zeroed
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    a[t] &= (2 * t >= lead ? 0xffffu : 0u) | (2 * t + 1 >= lead ? 0xffff0000u : 0u);
            }
            S = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, qB[j]), S,
                                                       0, 0, 0);
        }
        // the next tile's K, into the registers the MFMAs have just read
        const int kn = k0 + 32 * kWaves;
        band(kn);
        page = tile_page(kn);
        kload(kn, page, ka);

        // register r of half h holds key k0 + 16(r/8) + 8h + (r%8) for column l32
        if (tail) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (k0 + 16 * (r >> 3) + 8 * h + (r & 7) >= key_hi) S[r] = -INFINITY;
        }
        float mx = S[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
        mx = fmaxf(mx, xchg32(mx, xaddr));
        const float m_new = fmaxf(m, mx);
        if (__any(m_new > m + kTau)) {
            const float alpha = __builtin_amdgcn_exp2f(m - m_new);
            lsum *= alpha;
#pragma unroll
            for (int i = 0; i < NDB; ++i) O[i] *= alpha;
            m = m_new;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            S[r] = __builtin_amdgcn_exp2f(S[r] - m);
            lsum += S[r];
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const u32x4 pb = u32x4{pack_bf16x2(S[8 * c + 0], S[8 * c + 1]),
                                   pack_bf16x2(S[8 * c + 2], S[8 * c + 3]),
                                   pack_bf16x2(S[8 * c + 4], S[8 * c + 5]),
                                   pack_bf16x2(S[8 * c + 6], S[8 * c + 7])};
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                u32x4 a = va[c][db];
                if (tail) {                           // cache slots past kv_len: zero them
                    const int kb = k0 + 16 * c + 8 * h;
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        a[t] &= (kb + 2 * t < key_hi ? 0xffffu : 0u) | (kb + 2 * t + 1 < key_hi ? 0xffff0000u : 0u);
                }
                O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, pb), O[db], 0, 0, 0);
            }
        }
        // the next tile's V, into the registers the MFMAs have just read
        vload(kn, page, va);
        k0 = kn;
    }

    // this wave's (O^T, m, l) for its columns (q heads) into LDS: lane = column l32,
    // register r of dim block db is dim 32db + 8(r/4) + 4h + (r%4)
    const float l_tot = lsum + xchg32(lsum, xaddr);
    if (l32 < G) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sO[w][l32][32 * db + 8 * (r >> 2) + 4 * h + (r & 3)] = O[db][r];
        if (h == 0) {
            sO[w][l32][D] = m;
            sO[w][l32][D + 1] = l_tot;
        }
    }
    __syncthreads();

    // merge the 4 waves and write this item's partial (O relative to M, M, l)
    float* dst = p.partial + ((int64_t)bg * p.n_chunks + chunk) * G * (D + 2);
    for (int i = tid; i < G * D; i += blockDim.x) {
        const int hh = i / D, e = i % D;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sO[ww][hh][D]);
        float o = 0.f, ls = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float f = __builtin_amdgcn_exp2f(sO[ww][hh][D] - M);
            o += f * sO[ww][hh][e];
            ls += f * sO[ww][hh][D + 1];
        }
        dst[hh * (D + 2) + e] = o;
        if (e == 0) {
            dst[hh * (D + 2) + D] = M;
            dst[hh * (D + 2) + D + 1] = ls;
        }
    }
    if (p.counter) {
        uint64_t tot = cnt;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o);
        if (lane == 0 && tot) atomicAdd(p.counter, (unsigned long long)(tot * (uint64_t)G));
    }
}

// out[b][hq] = merge over the chunks c < ceil(kv_len/chunk) of the partials.
// Block = 256 threads = 8 chunk groups x 32 dims; grid = (B*Hq) x (D/32).
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p, Tables tab) {
    __shared__ float red[256];
    __shared__ float sacc[8][33];
    const int tid = threadIdx.x;
    const int bh = blockIdx.x, slice = blockIdx.y;
    const int b = bh / p.Hq, hq = bh % p.Hq;
    const int G = p.Hq / p.Hkv;
    const int g = hq / G, hh = hq % G;
    const int64_t Lb = clamp_len(p.kv_len[b], p.Lmax);
    const int nc = p.balanced ? byte_split<D>(p, tab, g).chunks_used(Lb)
                              : (int)((Lb + p.chunk - 1) / p.chunk);        // <= n_chunks
    if (nc == 0) {
        // no keys (kv_len <= 0): nothing to attend to; out = 0, lse = -inf
        if (tid < 32) {
            const int64_t oi = ((int64_t)b * p.Hq + hq) * D + slice * 32 + tid;
            if (p.out_f32) static_cast<float*>(p.out)[oi] = 0.f;
            else static_cast<uint16_t*>(p.out)[oi] = 0;
            if (p.lse && slice == 0 && tid == 0) p.lse[(int64_t)b * p.Hq + hq] = -INFINITY;
        }
        return;
    }
    const float* base = p.partial + ((int64_t)(b * p.Hkv + g) * p.n_chunks) * G * (D + 2) + hh * (D + 2);
    const int64_t cstride = (int64_t)G * (D + 2);

    float M = -INFINITY;
    for (int c = tid; c < nc; c += 256) M = fmaxf(M, base[c * cstride + D]);
    red[tid] = M;
    __syncthreads();
    for (int s = 128; s >= 1; s >>= 1) {
        if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
        __syncthreads();
    }
    M = red[0];
    __syncthreads();

    const int dl = tid & 31, grp = tid >> 5;
    const int e = slice * 32 + dl;
    float o = 0.f, ls = 0.f;
    for (int c = grp; c < nc; c += 8) {
        const float* pc = base + c * cstride;
        const float f = exp2f(pc[D] - M);
        o += f * pc[e];
        ls += f * pc[D + 1];
    }
    sacc[grp][dl] = o;
    if (dl == 0) sacc[grp][32] = ls;
    __syncthreads();
    if (tid < 32) {
        float ot = 0.f, lt = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ot += sacc[i][tid];
            lt += sacc[i][32];
        }
        const float r = ot / lt;
        const int64_t oi = ((int64_t)b * p.Hq + hq) * D + slice * 32 + tid;
        if (p.out_f32) static_cast<float*>(p.out)[oi] = r;
        else static_cast<uint16_t*>(p.out)[oi] = f32_to_bf16_bits(r);
        if (p.lse && slice == 0 && tid == 0)
            p.lse[(int64_t)b * p.Hq + hq] = (M + log2f(lt)) * 0.6931471805599453f;
    }
}

template <int D>
hipError_t launch_decode_d(const DecodeParams& p, const Tables& t, hipStream_t s) {
    dim3 grid((unsigned)((int64_t)p.n_chunks * p.B * p.Hkv)), block(64 * kWaves);
    if (p.pg.table) decode_partial_kernel<D, true><<<grid, block, 0, s>>>(p, t);
    else decode_partial_kernel<D, false><<<grid, block, 0, s>>>(p, t);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid2((unsigned)(p.B * p.Hq), D / 32), block2(256);
    decode_combine_kernel<D><<<grid2, block2, 0, s>>>(p, t);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, const Tables& t, hipStream_t s) {
    return p.d == 64 ? launch_decode_d<64>(p, t, s) : launch_decode_d<128>(p, t, s);
}

hipError_t decode_scratch(void** ptr) {
    // device address of `scratch` on the current device, looked up on the first call made
    // with that device current and kept per device (two threads racing on a first call
    // both store the same address)
    constexpr int kMaxDevices = 64;
    static std::atomic<void*> addr[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* a = addr[dev].load(std::memory_order_acquire);
    if (!a) {
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!a) return hipErrorInvalidSymbol;
        addr[dev].store(a, std::memory_order_release);
    }
    *ptr = a;
    return hipSuccess;
}

}  // namespace wpa

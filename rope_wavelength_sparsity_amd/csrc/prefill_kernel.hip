// Causal prefill with a per-RoPE-wavelength window (ATFlash abstract; WavePrune
// original abstract), on gfx950 MFMA: q.k in half precision, P*V in bf16.
//
// Work decomposition
//   A workgroup owns one (sequence b, kv head g, chunk of Gc q heads of that kv head) and
//   32*R consecutive query rows; compute wave w handles q head (w % Gc) and the 32 rows of
//   row group (w / Gc).  One more wave, the producer, streams key tiles (BN keys) into a
//   two-stage LDS ring with direct global->LDS loads, walking from the diagonal outward:
//   tile t+1 streams in while the compute waves, sharing each tile (GQA reuse), work on
//   tile t.  At d=64 a compute wave fits 128 VGPRs, so a CU runs two workgroups.
//
// Per 32x32 (query x key) sub-tile
//   Distance band: dmin/dmax over the sub-tile's visible elements.  With the window table
//   W (non-decreasing in the pair index), pairs split into dead (W < dmin), straddling
//   (dmin <= W < dmax) and fully active (W >= dmax).  Because the active pairs at any
//   distance are a suffix of the pair axis (ATFlash abstract: the kept terms form a
//   contiguous part of the contraction axis), fully active pairs occupy a suffix of 16-dim
//   blocks:
//     * S^T = K'_blk * Q'_blk^T on v_mfma_f32_32x32x16_f16 over those blocks only; the
//       leading pairs of the first such block are zeroed in the Q operand;
//     * straddling pairs are added per element on VALU with the exact test D <= W_i.
//   Sub-tiles are visited in order of growing distance, so both band edges only move
//   forward along the pair axis: they are tracked with running indices, not searched.
//   Scores are in log2 units (scale*log2 e is folded into Q), and the chain starts from
//   -m, the running row max, supplied by one more MFMA step, so the MFMA yields the
//   exponent of exp2 directly.  m only moves when a sub-tile's probabilities would sum past
//   2^9 (a wave-wide vote on the row sums; the row max across lane halves is formed only
//   then), which leaves the result exact.  Then causal mask, exp2, the row sum of the
//   bf16 probabilities (two small MFMAs) and O^T += V^T P^T on MFMA.
//
// Register layouts (32x32x16 MFMA: A row m and B column n live in lane m%32 / n%32, the
// 16-deep contraction is split 8+8 between lane halves; C element (row 8(r/4)+4(l/32)+r%4,
// column l%32) is register r of lane l):
//   Q operand (B): lane = query row, half h holds the first-half (h=0) or second-half
//     (h=1) components of the block's 8 pairs.
//   K operand (A): lane m%32 reads key row perm(m) = m with bits 2 and 3 swapped, so S^T
//     register r of half h holds key 16(r/8) + 8h + (r%8).  Registers 8c..8c+7 are then
//     exactly the 8 keys that half h must supply as the B operand of the P*V step over
//     keys 16c..16c+15, and the P^T operand needs no data movement.
//   V operand (A of the P*V step): 16 bytes per lane, the 8 keys of one key octet for one
//     dim.  A tile's values sit in LDS as in memory, by key octets ([BN/8][d][8]: lane l of
//     half h reads dim l%32 of octet 2c+h, 512 contiguous bytes per half, conflict-free),
//     so a tile is one contiguous block to copy from the workspace or the decode cache.
//   O^T accumulator: lane = query row, so the softmax rescale is a per-lane scalar.
#include <atomic>
#include <type_traits>

#include "wpa_device.hpp"
#include "wpa_internal.hpp"

namespace wpa {

namespace {

constexpr float kSumTau = 512.0f;  // lazy rescale: a row's probabilities may sum to 2^9

typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ inline int perm_row(int m) {
    return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ inline int key_of_reg(int r, int h) {
    return 16 * (r >> 3) + 8 * h + (r & 7);
}

__device__ inline uint32_t sel4(u32x4 v, int i) {
    uint32_t a = (i & 1) ? v[1] : v[0];
    uint32_t b = (i & 1) ? v[3] : v[2];
    return (i & 2) ? b : a;
}

// Exchange with lane l ^ 32 through ds_bpermute; `xaddr` = 4 * (lane ^ 32), computed once.
__device__ inline uint32_t partner32(uint32_t v, int xaddr) {
    return (uint32_t)__builtin_amdgcn_ds_bpermute(xaddr, (int)v);
}

__device__ inline float max_with_partner(float v, int xaddr) {
    return fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(xaddr, __builtin_bit_cast(int, v))));
}

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Leading nz pairs of an 8-pair block zeroed, as a mask on the packed block.
__device__ inline u32x4 lead_mask(int nz) {
    u32x4 q;
#pragma unroll
    for (int t = 0; t < 4; ++t)
        q[t] = ((2 * t >= nz) ? 0xffffu : 0u) | ((2 * t + 1 >= nz) ? 0xffff0000u : 0u);
    return q;
}

// The element e of an 8-pair block alone (both halves), as a mask on the packed block.
__device__ inline u32x4 pair_mask(int e) {
    u32x4 q;
#pragma unroll
    for (int t = 0; t < 4; ++t)
        q[t] = (e >> 1) == t ? ((e & 1) ? 0xffff0000u : 0xffffu) : 0u;
    return q;
}

// Number of registers r of a sub-tile with off(r) = 16(r/8) + r%8 <= x.
__device__ inline int n_off_le(int x) {
    const int a = x + 1 < 0 ? 0 : (x + 1 > 8 ? 8 : x + 1);
    const int b = x - 15 < 0 ? 0 : (x - 15 > 8 ? 8 : x - 15);
    return a + b;
}

// f(std::integral_constant<int, v>{}) for a run-time v in [0, N).
template <int N, class F>
__device__ inline void dispatch(int v, F&& f) {
    if constexpr (N > 0) {
        if (v == N - 1) f(std::integral_constant<int, N - 1>{});
        else dispatch<N - 1>(v, f);
    }
}

struct Launch {
    int Gc, R, nhc, n_rb;
    int ns;        // CACHED: key splits per row block (1: none; >1: partials in p.part)
};

template <int D>
struct Tile {
    static constexpr int BN = 128;                  // keys per tile (d=128: 64 was 5% slower)
    static constexpr int NSUB = BN / 32;
    static constexpr int KI = BN * 32 / 1024;       // wave loads per K block
    static constexpr int VI = D * BN * 2 / 1024;    // wave loads for V (1 KB each)
    static constexpr int PI = BN * 4 / 256;         // wave loads for positions
    // Compute waves per workgroup (plus one producer wave) and the waves per SIMD the
    // register budget must allow.  d=64 fits 128 VGPRs: 4 waves per SIMD, two 8-wave
    // workgroups per CU (64 KB of LDS each).  d=128 fits 168: 3 per SIMD, one 12-wave
    // workgroup per CU; with explicit positions (more registers) 2 per SIMD, 8 waves.
    static constexpr int maxw(bool haspos) { return D == 64 || haspos ? 7 : 11; }
    static constexpr int waves_per_eu(bool haspos) { return D == 64 ? 4 : (haspos ? 2 : 3); }
};

// CACHED: the keys and values are the decode caches (K pair-blocked with row stride
// ldk = Lmax, V blocked by key octets) and sequence b holds kv_len[b] of them; its Nq
// queries are its last Nq tokens (chunked prefill).  Positions are token indices.
// SPARSE: each (sequence, q head, 64-row query block) attends, besides its own block, only
// the 64-key blocks its ascending list names (token-level block sparsity composed with the
// window); unlisted keys leave the softmax.  Blocks are by token index; with HASPOS the
// rotation and the window use the explicit positions.
// HEADS: one rotation-frequency table per kv head (p.head_theta [Hkv][d/2], device); the
// workgroup's window table is computed from its kv head's row at start.
template <int D, bool F32, bool HASPOS, bool COUNT, bool CACHED, bool SPARSE, bool PAGED = false,
          bool HEADS = false>
__global__ __launch_bounds__(64 * (Tile<D>::maxw(HASPOS) + 1))
__attribute__((amdgpu_waves_per_eu(Tile<D>::waves_per_eu(HASPOS))))
void prefill_kernel(PrefillParams p, Tables tab, Launch L) {
    constexpr int NB = D / 16;
    constexpr int P = D / 2;
    constexpr int NDB = D / 32;
    constexpr int BN = Tile<D>::BN;
    constexpr int NSUB = Tile<D>::NSUB;
    __shared__ __attribute__((aligned(16))) uint16_t sK2[2][NB * BN * 16];
    __shared__ __attribute__((aligned(16))) uint16_t sV2[2][D * BN];
    __shared__ __attribute__((aligned(16))) int32_t sPos2[2][HASPOS ? BN : 1];
    extern __shared__ uint32_t sBits[];       // SPARSE: block bitmaps (dynamic size)

    const int tid = threadIdx.x;
    // wave index through readfirstlane: everything derived from it (head, rows, band
    // edges, branches on them) is then known to be wave-uniform and stays scalar
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, h = lane >> 5;
    const int xaddr = (lane ^ 32) << 2;
    const int G = p.Hq / p.Hkv;
    const int U = p.B * p.Hkv * L.nhc;
    const int u = blockIdx.x % U;
    // workgroup order: row blocks longest first, then their key splits, then (sequence, kv
    // head, head chunk)
    const int split = CACHED ? (int)(blockIdx.x / U) % L.ns : 0;
    const int rb = L.n_rb - 1 - (int)(blockIdx.x / U) / (CACHED ? L.ns : 1);
    const int hc = u % L.nhc;
    const int g = (u / L.nhc) % p.Hkv;
    const int b = u / (L.nhc * p.Hkv);
    // Window and rotation tables: the launch's (kernel arguments), or with per-head tables the
    // row of kv head g, its windows computed here once per workgroup (into LDS)
    __shared__ int32_t sWh[HEADS ? D / 2 : 1];
    if constexpr (HEADS) {
        if (tid < D / 2) sWh[tid] = window_from_theta(p.alpha, p.head_theta[(int64_t)g * (D / 2) + tid]);
        __syncthreads();
    }
    auto Wt = [&](int i) -> int {
        if constexpr (HEADS) return uniform(sWh[i]);
        else return tab.W[i];
    };
    auto TH = [&](int i) -> double {
        if constexpr (HEADS) return p.head_theta[(int64_t)g * (D / 2) + i];
        else return tab.theta[i];
    };
    const int hin = hc * L.Gc + (w % L.Gc);
    const int rg = w / L.Gc;
    const bool head_ok = hin < G;
    const int hq = g * G + (head_ok ? hin : 0);
    // Token geometry: NK keys (tokens 0..NK-1); the NQ rows of q and out are tokens
    // tq0..NK-1.  Row groups start at multiples of 32 tokens, so the first sub-tile a wave
    // visits holds the diagonal of all its rows.  (Plain prefill: NK = NQ = N, tq0 = 0.)
    int NQ = CACHED ? p.Nq : (int)p.N;
    int64_t row0 = (int64_t)b * NQ;                    // first row of this sequence in q / out
    if constexpr (CACHED) {
        if (p.cu_q) {
            // varlen: rows cu_q[b] .. cu_q[b+1]-1 of the packed q / out (at most Nq of them)
            const int c0 = uniform(p.cu_q[b]), c1 = uniform(p.cu_q[b + 1]);
            NQ = c1 - c0 < 0 ? 0 : (c1 - c0 > p.Nq ? p.Nq : c1 - c0);
            row0 = c0;
            if (NQ == 0) return;
        }
    }
    const int N_SP = (int)p.N;
    int NK = (int)p.N;
    if constexpr (CACHED) {
        NK = uniform(p.kv_len[b]);                     // in [Nq, Lmax] by contract; clamped
        NK = NK < NQ ? NQ : (NK > (int)p.N ? (int)p.N : NK);     // so that no access leaves
    }                                                  // the caches
    const int tq0 = NK - NQ;
    const int qs = (CACHED ? (tq0 & ~31) : 0) + rb * 32 * L.R;
    if (CACHED && qs >= NK) return;                    // this sequence has fewer rows
    const int row_end = (qs + 32 * L.R < NK ? qs + 32 * L.R : NK) - 1;
    // Key tiles 0 .. kt_last reach this workgroup's rows.  With key splits, split s of the row
    // block takes tiles [T s / ns, T (s+1) / ns) of those T and writes its share for the
    // combine: its rows' output normalised by their own sum over its keys, and m + log2 of
    // that sum.  A row block whose tiles all fall to one split (T = 1) writes its rows directly.
    int kt_last = row_end / BN, kt_lo = 0;
    bool partial = false;
    if constexpr (CACHED) {
        if (L.ns > 1) {
            const int T = kt_last + 1;
            kt_lo = (int)((int64_t)T * split / L.ns);
            const int hi = (int)((int64_t)T * (split + 1) / L.ns);
            if (kt_lo >= hi) return;                   // an empty split (T < ns)
            kt_last = hi - 1;
            partial = T > 1;
        }
    }
    const int q0 = qs + 32 * rg;
    const bool producer = w == L.Gc * L.R;                 // the extra, loading wave
    const bool wave_ok = !producer && head_ok && q0 < NK && (!CACHED || q0 + 31 >= tq0);
    const int qrow = q0 + l32;                             // this lane's row, as a token
    const bool row_ok = (!CACHED || qrow >= tq0) && qrow < NK;
    const int qrow_c = row_ok ? qrow : (CACHED && qrow < tq0 ? tq0 : NK - 1);
    const int qi = qrow_c - tq0;                           // ... and as a row of q / out
    const int32_t* posb = p.pos + (HASPOS ? (int64_t)b * NK : 0);
    auto POS = [&](int t) -> int { return HASPOS ? posb[t] : t; };
    const int pq = POS(qrow_c);

    // Scores are kept in log2 units: the softmax scale times log2(e) is folded into Q.
    const float sl2 = p.scale * 1.4426950408889634f;

    // ---- Q: load, round to bf16, rotate at its own position, scale, round to half (the
    // B operand of the q.k product)
    // All NB blocks as one vector value (not an array): a run-time block index then reads
    // registers, where an array would be moved to scratch memory.
    typedef uint32_t u32xQ __attribute__((ext_vector_type(4 * NB)));
    u32xQ Qv;
    auto Qf = [&](int j) -> u32x4 { return u32x4{Qv[4 * j], Qv[4 * j + 1], Qv[4 * j + 2], Qv[4 * j + 3]}; };
    {
        const int64_t qb = ((row0 + qi) * p.Hq + hq) * D;
        // the row's components as bf16 bits, first components (xw) and second components (yw)
        // of all pairs, packed two to a word: 16-byte loads issued for every block up front
        // (per-element loads inside the rotation loop made a chain of dependent round trips,
        // the fixed cost of every launch)
        u32x4 xw[NB], yw[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            if constexpr (F32) {
                float a[8], c[8];
                // pairs 8j..8j+7: (i, i+P) half-split, (2i, 2i+1) interleaved
                load8<true>(p.q, p.interleaved ? qb + 16 * j : qb + 8 * j, a);
                load8<true>(p.q, p.interleaved ? qb + 16 * j + 8 : qb + P + 8 * j, c);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    if (p.interleaved) {
                        const float* e = t < 2 ? a + 4 * t : c + 4 * (t - 2);
                        xw[j][t] = f32_to_bf16_bits(e[0]) | ((uint32_t)f32_to_bf16_bits(e[2]) << 16);
                        yw[j][t] = f32_to_bf16_bits(e[1]) | ((uint32_t)f32_to_bf16_bits(e[3]) << 16);
                    } else {
                        xw[j][t] = f32_to_bf16_bits(a[2 * t]) | ((uint32_t)f32_to_bf16_bits(a[2 * t + 1]) << 16);
                        yw[j][t] = f32_to_bf16_bits(c[2 * t]) | ((uint32_t)f32_to_bf16_bits(c[2 * t + 1]) << 16);
                    }
                }
            } else {
                const uint16_t* qh = static_cast<const uint16_t*>(p.q);
                const u32x4 a = *reinterpret_cast<const u32x4*>(qh + (p.interleaved ? qb + 16 * j : qb + 8 * j));
                const u32x4 c = *reinterpret_cast<const u32x4*>(qh + (p.interleaved ? qb + 16 * j + 8 : qb + P + 8 * j));
                if (p.interleaved) {
                    // word t of a (c) holds pair 8j+t (8j+4+t) as (x, y)
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const uint32_t lo = t < 2 ? a[2 * t] : c[2 * t - 4];
                        const uint32_t hi = t < 2 ? a[2 * t + 1] : c[2 * t - 3];
                        xw[j][t] = (lo & 0xffffu) | (hi << 16);
                        yw[j][t] = (lo >> 16) | (hi & 0xffff0000u);
                    }
                } else {
                    xw[j] = a;
                    yw[j] = c;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            // pairs 8j..8j+7, one at a time (rolled loop: one sincos instance per block);
            // each 16-bit result enters at the top of the 128-bit block value, which shifts
            // down by 16 bits, so after 8 steps pair 8j+e sits in element e.
            u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll 1
            for (int e = 0; e < 8; ++e) {
                const int sh = (e & 1) * 16;
                const float x = bf16_bits_to_f32((sel4(xw[j], e >> 1) >> sh) & 0xffffu);
                const float y = bf16_bits_to_f32((sel4(yw[j], e >> 1) >> sh) & 0xffffu);
                float sn, cs;
                rope_sincos(pq, TH(8 * j + e), &sn, &cs);
                const float rot = h ? (y * cs + x * sn) : (x * cs - y * sn);
                const uint32_t bits = f32_to_f16_bits(rot * sl2);
                acc[0] = (acc[0] >> 16) | (acc[1] << 16);
                acc[1] = (acc[1] >> 16) | (acc[2] << 16);
                acc[2] = (acc[2] >> 16) | (acc[3] << 16);
                acc[3] = (acc[3] >> 16) | (bits << 16);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) Qv[4 * j + t] = acc[t];
        }
    }

    const int64_t ldk = CACHED ? p.ldk : p.Np;            // key row stride of kp
    const uint16_t* kpg = p.kp + ((int64_t)b * p.Hkv + g) * NB * ldk * 16;
    // V by key octets: [Np/8][d][8] per head (plain) or the cache [ceil(Lmax/8)][d][8]
    const uint16_t* vtg = p.vt + ((int64_t)b * p.Hkv + g) * D *
                                     (CACHED ? (p.ldk + 7) / 8 * 8 : p.Np);
    const int pq_wg = POS(qs < NK ? qs : NK - 1);
    const int pq_lo = POS(q0 < NK ? q0 : NK - 1);
    const int pq_hi = POS(q0 + 31 < NK ? q0 + 31 : NK - 1);

    f32x16 O[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) O[i] = f32x16{};
    // Running row max m (log2 units) and sum.  The first sub-tile a wave visits holds the
    // diagonal of all its rows, so m is finite from then on; later score accumulators
    // start at -m, so the MFMA yields the exponent of exp2 directly.  The -m start is one
    // more MFMA step: a constant A block with 1 and 2048 in its first two columns (lanes of
    // half 0) against a B block holding -lo and -hi per query, m = 2048*hi + lo with hi, lo
    // half-precision values (m is kept at exactly that value; |m| < 1.3e8).
    float m = 0.f, lsum = 0.f;
    bool started = false;
    const u32x4 ones_blk = h ? u32x4{0u, 0u, 0u, 0u} : u32x4{0x68003c00u, 0u, 0u, 0u};   // (1, 2048)
    u32x4 negm_blk = {0u, 0u, 0u, 0u};
    // When the chain's first block has zeroed leading pairs, the -m step rides in it instead:
    // slot 0 of that block (pair 8jf: its first dim in half 0, its second in half 1) holds 2048
    // resp. 1 in the K operand and -hi resp. -lo in the Q operand (the pair's own term is then
    // not in this MFMA, which it must not be anyway).  One MFMA less per sub-tile for two VALU
    // bit merges: 2.6% faster at d=64, ~1% at d=128.
    const uint32_t kfold = h ? 0x3c00u : 0x6800u;            // 1, 2048 (half)
    uint32_t qfold = 0u;                                      // -lo, -hi (half)
    auto set_m = [&](float mv) {
        const _Float16 hi = (_Float16)(mv * (1.0f / 2048.0f));
        const _Float16 lo = (_Float16)(mv - 2048.0f * (float)hi);
        m = 2048.0f * (float)hi + (float)lo;
        const uint32_t nlo = __builtin_bit_cast(uint16_t, (_Float16)-lo);
        const uint32_t nhi = __builtin_bit_cast(uint16_t, (_Float16)-hi);
        negm_blk[0] = h ? 0u : (nlo | (nhi << 16));
        qfold = h ? nlo : nhi;
    };
    uint64_t cnt = 0;
    int plo = 0, pfull = 0, plo_wg = 0;     // running band edges (distances only grow)
    int w_lo = Wt(0), w_full = Wt(0);  // W at the two edges (INT32_MAX past the end)
    // Block jf = pfull/8 of Q with its leading (not fully active) pairs zeroed, valid for
    // the band edge pfull == q_key; rebuilt only when that edge moves.
    // kept in LDS (one slot per lane of each compute wave), not in registers
    __shared__ u32x4 sQm[Tile<D>::maxw(false) > Tile<D>::maxw(true) ? Tile<D>::maxw(false) : Tile<D>::maxw(true)][64];
    auto set_qm = [&](u32x4 v) { sQm[w][lane] = v; };
    auto qm = [&]() { return sQm[w][lane]; };
    int q_key = -1;

    // Stream key tile kt into `stage` with direct global->LDS loads (one wave instruction
    // fills 1 KB of LDS: lane l's bytes land at base + size*l).  Only the pair blocks that
    // can be active anywhere in the tile (from the workgroup's smallest distance) are read.
    // Paged caches: the page-table entries of the next tile to copy, read one tile ahead (a
    // lookup right before the copies made a dependent round trip per tile).
    int32_t pgs[BN / 32] = {};
    auto fetch_pages = [&](int kt) {
        if constexpr (CACHED && PAGED) {
            const int ks = kt * BN, lg = p.pg.page_log2;
            if ((1 << lg) >= BN) {
                pgs[0] = uniform((int)page_of(p.pg, b, ks));
            } else {
#pragma unroll
                for (int i = 0; i < BN / 32; ++i) {
                    const int t = ks + (i << lg);
                    pgs[i] = (t < ks + BN) ? uniform((int)page_of(p.pg, b, t < NK ? t : NK - 1)) : 0;
                }
            }
        }
    };
    auto issue = [&](int kt, int stage) {
        const int ks = kt * BN;
        const int kend = (ks + BN < NK ? ks + BN : NK) - 1;
        const int dmin_wg = uniform(pq_wg - POS(kend) > 0 ? pq_wg - POS(kend) : 0);
        while (plo_wg < P && Wt(plo_wg) < dmin_wg) ++plo_wg;
        const int jlo = uniform(plo_wg) >> 3;
        const int nK = Tile<D>::KI * (NB - jlo);
        const int nI = nK + Tile<D>::VI + (HASPOS ? Tile<D>::PI : 0);
        // paged caches: the tile's page when a page holds whole tiles (page_size >= BN), else
        // the pages of its BN / page_size page slots (at most 4: pages hold >= 32 tokens),
        // fetched by the previous call (fetch_pages) while its copies were in flight
        constexpr bool paged = CACHED && PAGED;
        const bool small_pages = paged && (1 << p.pg.page_log2) < BN;
        // page of token t of this tile (t in [ks, ks + BN))
        auto page_at = [&](int t) -> int64_t {
            if (!small_pages) return pgs[0];
            const int slot = (t - ks) >> p.pg.page_log2;
            int32_t pg_ = pgs[0];
#pragma unroll
            for (int i = 1; i < BN / 32; ++i) pg_ = slot == i ? pgs[i] : pg_;
            return pg_;
        };
        if constexpr (!CACHED) {
            // One-shot prefill: block j of the tile is KI contiguous 1 KB pieces and V is one
            // contiguous run of VI pieces, so each copy is a scalar base plus constant offsets
            // (the per-load address arithmetic ran on the scalar unit every compute wave of the
            // CU shares).
            const uint16_t* kb = kpg + ((int64_t)jlo * ldk + ks) * 16 + lane * 8;
            for (int j = jlo; j < NB; ++j, kb += ldk * 16) {
#pragma unroll
                for (int part = 0; part < Tile<D>::KI; ++part)
                    __builtin_amdgcn_global_load_lds(kb + part * 512,
                                                     (lds_ptr)&sK2[stage][j * BN * 16 + part * 512], 16, 0, 0);
            }
            const uint16_t* vb = vtg + (int64_t)ks * D + lane * 8;
#pragma unroll
            for (int r = 0; r < Tile<D>::VI; ++r)
                __builtin_amdgcn_global_load_lds(vb + r * 512, (lds_ptr)&sV2[stage][r * 512], 16, 0, 0);
            if constexpr (HASPOS) {
#pragma unroll
                for (int pi = 0; pi < Tile<D>::PI; ++pi) {
                    const int t = ks + 64 * pi + lane;
                    __builtin_amdgcn_global_load_lds(posb + (t < NK ? t : NK - 1),
                                                     (lds_ptr)&sPos2[stage][64 * pi], 4, 0, 0);
                }
            }
            return;
        }
        if constexpr (CACHED) {
            if (ks + BN <= NK) {
                // a tile with no key past the last: 32-token K pieces and V pieces (one octet, or
                // half of one at d=128) each lie in one page, so every copy is a scalar base plus
                // the lane's 16 bytes, as in the one-shot prefill
                const int lg = p.pg.page_log2, ps = 1 << lg;
                for (int j = jlo; j < NB; ++j) {
#pragma unroll
                    for (int part = 0; part < Tile<D>::KI; ++part) {
                        const uint16_t* kb;
                        if constexpr (paged) {
                            const int64_t pg_ = small_pages ? pgs[(part * 32) >> lg] : pgs[0];
                            kb = p.kp + (((pg_ * p.Hkv + g) * NB + j) * ps + ((ks + part * 32) & (ps - 1))) * 16;
                        } else {
                            kb = kpg + ((int64_t)j * ldk + ks + part * 32) * 16;
                        }
                        __builtin_amdgcn_global_load_lds(kb + lane * 8,
                                                         (lds_ptr)&sK2[stage][j * BN * 16 + part * 512], 16, 0, 0);
                    }
                }
#pragma unroll
                for (int r = 0; r < Tile<D>::VI; ++r) {
                    const int c = 64 * r / D;                 // the piece's octet in the tile
                    const uint16_t* vb;
                    if constexpr (paged) {
                        const int opg = ps >> 3;
                        const int64_t pg_ = small_pages ? pgs[(8 * c) >> lg] : pgs[0];
                        vb = p.vt + (((pg_ * p.Hkv + g) * opg + ((ks / 8 + c) & (opg - 1))) * D) * 8 +
                             (64 * r - c * D) * 8;
                    } else {
                        vb = vtg + (int64_t)(ks / 8) * D * 8 + 64 * r * 8;
                    }
                    __builtin_amdgcn_global_load_lds(vb + lane * 8, (lds_ptr)&sV2[stage][r * 512], 16, 0, 0);
                }
                if (kt > kt_lo) fetch_pages(kt - 1);
                return;
            }
        }
        for (int i = 0; i < nI; ++i) {
            if (i < nK) {
                // 16-byte chunk `ch` of block j: half (ch & 1) of key ks + ch/2 (past the last
                // key of a cache, the last key stands in: those keys are masked)
                const int j = jlo + i / Tile<D>::KI, part = i % Tile<D>::KI;
                const int ch = part * 64 + lane;
                const uint16_t* src;
                if constexpr (CACHED) {
                    int t = ks + (ch >> 1);
                    if (t > NK - 1) t = NK - 1;
                    if constexpr (paged) {
                        const int ps = 1 << p.pg.page_log2;
                        src = p.kp + (((page_at(t) * p.Hkv + g) * NB + j) * ps + (t & (ps - 1))) * 16 +
                              (ch & 1) * 8;
                    } else {
                        src = kpg + ((int64_t)j * ldk + t) * 16 + (ch & 1) * 8;
                    }
                } else {
                    src = kpg + ((int64_t)j * ldk + ks) * 16 + ch * 8;
                }
                __builtin_amdgcn_global_load_lds(src, (lds_ptr)&sK2[stage][j * BN * 16 + part * 512],
                                                 16, 0, 0);
            } else if (i < nK + Tile<D>::VI) {
                // the tile's octets as one block: 16-byte piece 64r + lane is dim e of
                // octet c (past the last key of a cache, its last octet stands in: those
                // keys are masked)
                const int r = i - nK;
                const int pc = 64 * r + lane, c = pc / D, e = pc % D;
                int o = ks / 8 + c;
                const uint16_t* src;
                if constexpr (CACHED) {
                    if (o > (NK - 1) / 8) o = (NK - 1) / 8;
                    if constexpr (paged) {
                        const int opg = 1 << (p.pg.page_log2 - 3);        // octets per page
                        src = p.vt + (((page_at(8 * o) * p.Hkv + g) * opg + (o & (opg - 1))) * D + e) * 8;
                    } else {
                        src = vtg + ((int64_t)o * D + e) * 8;
                    }
                } else {
                    src = vtg + ((int64_t)o * D + e) * 8;
                }
                __builtin_amdgcn_global_load_lds(src, (lds_ptr)&sV2[stage][r * 512], 16, 0, 0);
            } else if (HASPOS) {
                const int pi = i - nK - Tile<D>::VI;
                const int t = ks + 64 * pi + lane;
                const int32_t* src = posb + (t < NK ? t : NK - 1);
                __builtin_amdgcn_global_load_lds(src, (lds_ptr)&sPos2[stage][64 * pi], 4, 0, 0);
            }
        }
        if constexpr (CACHED) {
            // The tile past the last key (only the one holding key NK-1): once its loads have
            // landed, its V slots of keys >= NK (cache slots never written, or other data) are
            // set to zero, so that their zero probabilities give zero terms in P*V.
            if (ks + BN > NK) {
                __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
                const int first = NK - ks;             // first key slot to clear, in [1, BN)
                const int co = first >> 3, j0 = first & 7;
                for (int pc = co * D + lane; pc < (BN / 8) * D; pc += 64) {
                    u32x4* cell = reinterpret_cast<u32x4*>(&sV2[stage][pc * 8]);
                    if (pc / D > co || j0 == 0) {
                        *cell = u32x4{0u, 0u, 0u, 0u};
                    } else {
                        u32x4 x = *cell;
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            x[t] &= (2 * t < j0 ? 0xffffu : 0u) | (2 * t + 1 < j0 ? 0xffff0000u : 0u);
                        *cell = x;
                    }
                }
            }
            // the next tile's pages (tiles go kt_last down to kt_lo)
            if (kt > kt_lo) fetch_pages(kt - 1);
        }
    };

    // Softmax step and P*V of one sub-tile (keys k0 .. k0+31, `sub` within its tile):
    // probabilities relative to the running max m, packed to bf16 as P*V takes them, and
    // the row's sum of them over all 32 keys, on every lane of the row.
    // The sum comes from two 16x16x32 MFMAs that take the packed probabilities as their B
    // operand unchanged: there lane 32h + l32 holds query l32 % 16 + 16 (l32 / 16) in K
    // group 2h + l32 / 16, and the constant A operand `rsel` (ones in rows 0 and 8 over K
    // groups 0 and 2, in rows 4 and 12 over groups 1 and 3, zeros elsewhere) adds both
    // halves' groups of each query into the output row whose register 0 that query's lanes
    // hold.  (Eight dependent v_dot2 per sub-tile, half-row sums, were 8% slower in a
    // model of this loop.)
    // m moves only when the probabilities would grow past 2^9: every probability is at most
    // the row sum, so a wave-wide vote on that sum replaces a max over the scores.  The
    // rare sub-tile that fails it (and the first one, which sets m) recomputes its scores
    // and takes the row max.
    const uint32_t rsel_w = (((lane & 3) == 0) && ((((lane >> 2) ^ (lane >> 4)) & 1) == 0)) ? 0x3f803f80u : 0u;
    const bf16x8 rsel = __builtin_bit_cast(bf16x8, u32x4{rsel_w, rsel_w, rsel_w, rsel_w});
    auto probs = [&](const f32x16& S, uint32_t (&wd)[8]) -> float {
#pragma unroll
        for (int t = 0; t < 8; ++t)
            wd[t] = pack_bf16x2(__builtin_amdgcn_exp2f(S[2 * t]), __builtin_amdgcn_exp2f(S[2 * t + 1]));
        f32x4 R = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            rsel, __builtin_bit_cast(bf16x8, u32x4{wd[0], wd[1], wd[2], wd[3]}), f32x4{}, 0, 0, 0);
        R = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            rsel, __builtin_bit_cast(bf16x8, u32x4{wd[4], wd[5], wd[6], wd[7]}), R, 0, 0, 0);
        return R[0];
    };
    // scores S (relative to m; absolute before the first sub-tile) -> new m, O and the row
    // sum rescaled, S made relative to the new m
    auto remax = [&](f32x16& S) {
        float mx = S[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
        mx = max_with_partner(mx, xaddr);
        float shift;
        if (!started) {
            set_m(mx);
            shift = m;
            started = true;
        } else {
            const float m_old = m;
            set_m(m + fmaxf(mx, 0.f));
            shift = m - m_old;
            const float alpha = __builtin_amdgcn_exp2f(-shift);
            lsum *= alpha;
#pragma unroll
            for (int i = 0; i < NDB; ++i) O[i] *= alpha;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) S[r] -= shift;
    };
    const int v_lane = (h * D + l32) * 8;                    // dim l32 of octet h (db = 0, c = 0)
    auto pv = [&](int sub, const uint32_t (&wd)[8], const uint16_t* sV) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const u32x4 pb = u32x4{wd[4 * c], wd[4 * c + 1], wd[4 * c + 2], wd[4 * c + 3]};
            // keys 16(2sub + c) + 8h .. +7: octet 4sub + 2c + h of the tile
            const uint16_t* vp = sV + v_lane + (4 * sub + 2 * c) * D * 8;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(vp + 32 * db * 8);
                O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    a, __builtin_bit_cast(bf16x8, pb), O[db], 0, 0, 0);
            }
        }
    };
    auto bias = [&](const f32x16& S) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(
            __builtin_bit_cast(f16x8, ones_blk), __builtin_bit_cast(f16x8, negm_blk), S, 0, 0, 0);
    };

    // One key tile from LDS: its 32-key sub-tiles, nearest keys first.
    // kmask: bit i set = key block (ks/64 + i) of this tile is in this wave's list (SPARSE)
    auto compute = [&](int kt, const uint16_t* sK, const uint16_t* sV, const int32_t* sPos,
                       int kmask) {
        const int ks = kt * BN;
        constexpr int FULL = (1 << (BN / 64)) - 1;
        auto POSL = [&](int t) -> int { return uniform(HASPOS ? sPos[t - ks] : t); };

        // Plain tile: every key precedes every row of the wave (no causal mask), none is past
        // the last key, and no window edge falls inside the tile's distance range, so every
        // pair is dead or fully active on the whole tile.  The band is then fixed for the tile
        // and its sub-tiles run the chain of that block set, known at compile time.  The
        // tile's smallest distance is its nearest sub-tile's, so moving plo there is the step
        // that sub-tile would take anyway.
        bool plain = false;
        if (started && ks + BN - 1 < q0 && ks + BN <= NK && (!SPARSE || kmask == FULL)) {
            const int dmin_t = pq_lo - POSL(ks + BN - 1);
            const int dmax_t = pq_hi - POSL(ks);
            while (w_lo < dmin_t) {
                ++plo;
                w_lo = plo < P ? Wt(plo) : INT32_MAX;
            }
            if (w_lo >= dmax_t && plo < P) {
                pfull = plo;                    // no W in [dmin_t, dmax_t): plo is also the
                w_full = w_lo;                  // first pair active at dmax_t
                const int jf = pfull >> 3;
                if (pfull != q_key) {
                    set_qm(Qf(jf) & lead_mask(pfull - 8 * jf));
                    q_key = pfull;
                }
                if (COUNT && row_ok) cnt += (uint64_t)(16 * NSUB) * (uint64_t)(P - pfull);
                plain = true;
            }
        }
        const uint16_t* kl = sK + perm_row(l32) * 16 + 8 * h;   // this lane's K row (sub 0)

        // Scores of sub-tile `sub` without the -m step, on one MFMA chain: the fully active
        // blocks, preceded, when pairs straddle the window edge, by each such pair as its own
        // step (Q operand holding that pair alone), after which the elements outside its
        // window go back to zero.  Pair windows grow with the pair index, so an element
        // outside pair e's window is outside every earlier one's too and still holds zero:
        // the reset removes exactly pair e's term.  Then the causal mask.  Moves the band to
        // this sub-tile (sub-tiles come nearest first, so distances only grow) on the first
        // call for it (`count`), which also counts its kept terms.
        auto raw = [&](int sub, bool count) -> f32x16 {
            const int k0 = ks + 32 * sub;
            const uint16_t* ksub = kl + 32 * sub * 16;            // this lane's K row, this sub-tile
            auto K = [&](int j) { return *reinterpret_cast<const f16x8*>(ksub + j * BN * 16); };
            f32x16 S;
            // the first active block's operands, with the -m step folded in when it can be
            auto first = [&](int j, f32x16 acc) {
                const uint32_t fm = (pfull & 7) ? 0xffffu : 0u;
                u32x4 kj = __builtin_bit_cast(u32x4, K(j)), qj = qm();
                kj[0] = (kj[0] & ~fm) | (kfold & fm);
                qj[0] = (qj[0] & ~fm) | (qfold & fm);
                return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, kj),
                                                              __builtin_bit_cast(f16x8, qj), acc, 0, 0, 0);
            };
            if (plain) {
                // the tile's block set, unrolled for each first block
                dispatch<NB>(pfull >> 3, [&](auto jfc) {
                    constexpr int JF = decltype(jfc)::value;
                    f32x16 T = first(JF, f32x16{});
#pragma unroll
                    for (int j = JF + 1; j < NB; ++j)
                        T = __builtin_amdgcn_mfma_f32_32x32x16_f16(K(j), __builtin_bit_cast(f16x8, Qf(j)), T, 0, 0, 0);
                    S = T;
                });
                return S;
            }
            if (count) {
                // (a recomputation finds the band already at this sub-tile)
                const int k_last = k0 + 31 < NK ? k0 + 31 : NK - 1;
                const int dmin = pq_lo - POSL(k_last) > 0 ? pq_lo - POSL(k_last) : 0;
                const int dmax = pq_hi - POSL(k0);
                while (w_lo < dmin) {
                    ++plo;
                    w_lo = plo < P ? Wt(plo) : INT32_MAX;
                }
                while (w_full < dmax) {
                    ++pfull;
                    w_full = pfull < P ? Wt(pfull) : INT32_MAX;
                }
                const int jn = pfull >> 3;
                if (pfull != q_key && jn < NB) {
                    set_qm(Qf(jn) & lead_mask(pfull - 8 * jn));
                    q_key = pfull;
                }
            }
            const int jf = pfull >> 3;
            const bool diag = k0 + 31 > q0;
            // register r of half h holds key k0 + off(r) + 8h, off(r) = 16(r/8) + r%8:
            // causal iff off(r) <= lim
            const int lim = qrow - k0 - 8 * h;
            if (COUNT && count && row_ok) {
                // kept terms of this row: fully active pairs on every causal key, straddling
                // pairs on the causal keys inside their window
                const int nv = diag ? n_off_le(lim) : 16;
                cnt += (uint64_t)nv * (uint64_t)(P - pfull);
                for (int e = plo; e < pfull; ++e) {
                    if constexpr (HASPOS) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int kk = 32 * sub + key_of_reg(r, h);
                            cnt += (16 * (r >> 3) + (r & 7) <= lim && pq - sPos[kk] <= Wt(e)) ? 1 : 0;
                        }
                    } else {
                        const int c = n_off_le(lim) - n_off_le(lim - Wt(e) - 1);
                        cnt += c > 0 ? c : 0;
                    }
                }
            }

            auto upper = [&](f32x16 A) {        // the fully active blocks above jf
#pragma unroll
                for (int j = NB - 1; j >= 1; --j)
                    if (j > jf) A = __builtin_amdgcn_mfma_f32_32x32x16_f16(K(j), __builtin_bit_cast(f16x8, Qf(j)), A, 0, 0, 0);
                return A;
            };
            if (!HASPOS && plo < pfull) {
                f32x16 T = {};
#pragma unroll 1
                for (int e = plo; e < pfull; ++e) {
                    const u32x4 qe = Qf(e >> 3) & pair_mask(e & 7);
                    T = __builtin_amdgcn_mfma_f32_32x32x16_f16(K(e >> 3), __builtin_bit_cast(f16x8, qe), T, 0, 0, 0);
                    const int t = lim - Wt(e);              // inside iff off(r) >= t
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (16 * (r >> 3) + (r & 7) < t) T[r] = 0.f;
                }
                if (jf < NB) T = first(jf, T);
                S = upper(T);
            } else if (jf < NB) {
                S = upper(first(jf, f32x16{}));
            } else {
                S = f32x16{};
            }
            if constexpr (HASPOS) {
                // arbitrary positions: straddling pairs per element on VALU
                if (plo < pfull) {
#pragma unroll
                    for (int j = 0; j < NB; ++j) {
                        const int e_lo = plo - 8 * j > 0 ? plo - 8 * j : 0;
                        const int e_hi = pfull - 8 * j < 8 ? pfull - 8 * j : 8;
                        if (e_lo >= e_hi) continue;
                        const u32x4 mine = Qf(j);
                        u32x4 oth;
#pragma unroll
                        for (int t = 0; t < 4; ++t) oth[t] = partner32(mine[t], xaddr);
                        const u32x4 qx = h ? oth : mine;
                        const u32x4 qy = h ? mine : oth;
                        for (int e = e_lo; e < e_hi; ++e) {
                            const int sh = (e & 1) * 16;
                            const float fqx = f16_bits_to_f32((sel4(qx, e >> 1) >> sh) & 0xffffu);
                            const float fqy = f16_bits_to_f32((sel4(qy, e >> 1) >> sh) & 0xffffu);
                            const int Wi = Wt(8 * j + e);
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int kk = 32 * sub + key_of_reg(r, h);
                                const uint16_t* kr = &sK[(j * BN + kk) * 16];
                                const float kx = f16_bits_to_f32(kr[e]);
                                const float ky = f16_bits_to_f32(kr[8 + e]);
                                S[r] += (pq - sPos[kk] <= Wi) ? (fqx * kx + fqy * ky) : 0.f;
                            }
                        }
                    }
                }
            }
            // causal mask (raw scores; the scale is folded into the exponent)
            if (diag) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (16 * (r >> 3) + (r & 7) > lim) S[r] = -INFINITY;
            }
            return S;
        };

        // Sub-tiles above the diagonal, or past the last key, come first in the visiting
        // order and are skipped.
        int sub = NSUB - 1, sub_lo = 0;
        if (!plain) {
            const int a = (q0 + 31 - ks) >> 5, c = (NK - 1 - ks) >> 5;
            sub = a < sub ? a : sub;
            sub = uniform(c < sub ? c : sub);
            if constexpr (SPARSE) {
                // sub-tiles 2i, 2i+1 form key block i of the tile; the wave's blocks here are a
                // contiguous run of them
                if (kmask == 0) return;
                int hi = BN / 64 - 1;
                while (!((kmask >> hi) & 1)) --hi;
                int lo = 0;
                while (!((kmask >> lo) & 1)) ++lo;
                sub = 2 * hi + 1 < sub ? 2 * hi + 1 : sub;
                sub_lo = 2 * lo;
            }
        }
        if (sub < sub_lo) return;
        // The -m step of a sub-tile follows the previous sub-tile's vote, which may move m.  A
        // sub-tile that fails the vote recomputes its scores (the band still sits at it).  (Issuing
        // the next sub-tile's chain before this one's softmax cost the d=64 kernel 12 spilled
        // registers and 3%.)
        // the sub-tile index as top - i with a loop counter i: both scalar (a decremented index
        // merged from the two ways of computing its start lived in a vector register)
        const int sub_top = uniform(sub), n_sub = uniform(sub - sub_lo + 1);
#pragma unroll 1
        for (int i = 0; i < n_sub; ++i) {
            sub = sub_top - i;
            // the QK chain at raised wave priority: the SIMD's arbiter then issues each
            // dependent MFMA as soon as it can, and the other waves' softmax work fills the
            // gaps (2% faster at both d; raising P*V as well, or the producer, gained less)
            __builtin_amdgcn_s_setprio(1);
            const f32x16 T = raw(sub, true);
            // the -m step, unless the chain's first block carried it
            const bool folded = (pfull & 7) != 0 && (pfull >> 3) < NB;
            f32x16 S;
            if (folded) S = T;
            else S = bias(T);
            __builtin_amdgcn_s_setprio(0);
            uint32_t wd[8];
            float psum = 0.f;
            bool redo = !started;
            if (started) {
                psum = probs(S, wd);
                redo = __any(psum > kSumTau);
            }
            if (redo) {
                f32x16 R = raw(sub, false);
                if (!folded) R = bias(R);
                remax(R);
                psum = probs(R, wd);
            }
            lsum += psum;
            pv(sub, wd, sV);
        }
    };

    // The producer wave streams tile kt-1 into one stage while the others compute tile kt
    // from the other stage; it waits for its own loads before the barrier that hands the
    // stage over, so no compute wave ever has a direct load in flight (the compiler would
    // otherwise hold every LDS read of a compute wave until such loads land).
    if constexpr (!SPARSE) {
        if (producer) {
            fetch_pages(kt_last);
            issue(kt_last, 0);
            __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
        }
        for (int kt = kt_last, it = 0; kt >= kt_lo; --kt, ++it) {
            __syncthreads();          // tile kt is in stage it&1; stage (it+1)&1 is free again
            if (producer) {
                if (kt > kt_lo) {
                    issue(kt - 1, (it & 1) ^ 1);
                    __builtin_amdgcn_s_waitcnt(0x0070);
                }
            } else if (wave_ok) {
                compute(kt, sK2[it & 1], sV2[it & 1], sPos2[it & 1], 0);
            }
        }
    } else {
        // The lists as bitmaps in LDS: one bit per 64-key block for each compute wave and their
        // union.  A list block of 64 << s keys sets 1 << s consecutive bits (aligned, so never
        // across a word); the wave's own list block is always set up to its own 64-key block.
        const int nblk = (N_SP + 63) / 64, words = (nblk + 31) / 32;
        const int NL = L.Gc * L.R;
        uint32_t* uni = sBits + NL * words;
        for (int i = tid; i < (NL + 1) * words; i += blockDim.x) sBits[i] = 0u;
        __syncthreads();
        if (!producer && wave_ok) {
            const int s = p.blk_log2 - 6;
            const int rb = q0 >> 6, R = q0 >> p.blk_log2;
            const int nlb = (N_SP + (1 << p.blk_log2) - 1) >> p.blk_log2;
            uint32_t* mine = sBits + w * words;
            for (int t = (R << s) + lane; t <= rb; t += 64) {
                atomicOr(&mine[t >> 5], 1u << (t & 31));
                atomicOr(&uni[t >> 5], 1u << (t & 31));
            }
            const uint32_t run = (1u << (1 << s)) - 1u;        // s <= 4
            const int64_t li = ((int64_t)b * p.Hq + hq) * nlb + R;
            int c = p.blk_count[li];
            c = c < 0 ? 0 : (c > p.blk_max ? p.blk_max : c);
            for (int e = lane; e < c; e += 64) {
                const int kb = p.blk_idx[li * p.blk_max + e];
                if (kb >= 0 && kb < R) {
                    const int t = kb << s;
                    atomicOr(&mine[t >> 5], run << (t & 31));
                    atomicOr(&uni[t >> 5], run << (t & 31));
                }
            }
        }
        __syncthreads();
        // this compute wave's blocks of tile kt (tiles start at even blocks: no word straddle)
        auto wmask = [&](int kt) -> int {
            const int b0 = kt * BN / 64;
            return uniform((int)((sBits[w * words + (b0 >> 5)] >> (b0 & 31)) & ((1u << (BN / 64)) - 1u)));
        };
        // Every tile is visited (a loop jumping between needed tiles made the compiler keep
        // two copies of the accumulators); the producer loads only the needed ones, and a
        // compute wave returns at once from a tile without its blocks.
        auto needed = [&](int kt) {
            const int b0 = kt * BN / 64;
            return ((uni[b0 >> 5] >> (b0 & 31)) & ((1u << (BN / 64)) - 1u)) != 0u;
        };
        if (producer) {
            if (needed(kt_last)) issue(kt_last, 0);
            __builtin_amdgcn_s_waitcnt(0x0070);
        }
        for (int kt = kt_last, it = 0; kt >= 0; --kt, ++it) {
            __syncthreads();
            if (producer) {
                if (kt > 0 && needed(kt - 1)) {
                    issue(kt - 1, (it & 1) ^ 1);
                    __builtin_amdgcn_s_waitcnt(0x0070);
                }
            } else if (wave_ok) {
                compute(kt, sK2[it & 1], sV2[it & 1], sPos2[it & 1], wmask(kt));
            }
        }
    }

    if (COUNT) {
        uint64_t tot = cnt;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o);
        if (lane == 0 && wave_ok && tot) atomicAdd(p.counter, (unsigned long long)tot);
    }
    if (!wave_ok) return;
    const float l_tot = lsum;                  // the whole row's sum on both lanes of the row
    if (!row_ok) return;
    if (CACHED && partial) {
        // this split's share: rows with no key in its range hold sum 0 (output 0, log2-sum
        // -inf); the partials of split s sit at [s][b*Nq + qi][hq]
        const int64_t pr = ((int64_t)split * p.B * p.Nq + (int64_t)b * p.Nq + qi) * p.Hq + hq;
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        float* po = p.part + pr * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const int dim = 32 * db + 8 * grp + 4 * h;
                *reinterpret_cast<f32x4*>(po + dim) =
                    f32x4{O[db][4 * grp] * inv, O[db][4 * grp + 1] * inv, O[db][4 * grp + 2] * inv,
                          O[db][4 * grp + 3] * inv};
            }
        }
        if (h == 0)
            p.part[(int64_t)L.ns * p.B * p.Nq * p.Hq * D + pr] = l_tot > 0.f ? m + log2f(l_tot) : -INFINITY;
        return;
    }
    const float inv = 1.0f / l_tot;
    const int64_t ob = ((row0 + qi) * p.Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
            const int dim = 32 * db + 8 * grp + 4 * h;
            const float o0 = O[db][4 * grp + 0] * inv, o1 = O[db][4 * grp + 1] * inv;
            const float o2 = O[db][4 * grp + 2] * inv, o3 = O[db][4 * grp + 3] * inv;
            if (p.out_f32) {
                *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + ob + dim) =
                    f32x4{o0, o1, o2, o3};
            } else {
                uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.out) + ob + dim);
                dst[0] = pack_bf16x2(o0, o1);
                dst[1] = pack_bf16x2(o2, o3);
            }
        }
    }
    if (p.lse && h == 0)
        p.lse[CACHED && p.cu_q ? (row0 + qi) * p.Hq + hq : ((int64_t)b * p.Hq + hq) * NQ + qi] =
            (m + log2f(l_tot)) * 0.6931471805599453f;
}

// Merge of the key splits of a cached prefill: each (row, q head) of a row block with more
// than one key tile takes the splits that hold tiles of its row block (the same partition
// as the attention kernel's), weighs each by 2^(its log2-sum - their max), and writes the
// normalised sum and the natural-log lse.  D/4 threads per (row, head), 4 dims each.
template <int D>
__global__ __launch_bounds__(256) void split_combine(PrefillParams p, int R, int ns) {
    constexpr int BN = Tile<D>::BN, TPR = D / 4;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t pr = gid / TPR;                          // (b*Nq + qi)*Hq + hq
    const int c = (int)(gid % TPR);
    const int64_t npr = (int64_t)p.B * p.Nq * p.Hq;
    if (pr >= npr) return;
    const int hq = (int)(pr % p.Hq);
    const int64_t bq = pr / p.Hq;
    const int b = (int)(bq / p.Nq), qi = (int)(bq % p.Nq);
    // the sequence's geometry, as the attention kernel derives it
    int NQ = p.Nq;
    int64_t row0 = (int64_t)b * p.Nq;
    if (p.cu_q) {
        const int c0 = p.cu_q[b], c1 = p.cu_q[b + 1];
        NQ = c1 - c0 < 0 ? 0 : (c1 - c0 > p.Nq ? p.Nq : c1 - c0);
        row0 = c0;
    }
    if (qi >= NQ) return;
    int NK = p.kv_len[b];
    NK = NK < NQ ? NQ : (NK > (int)p.N ? (int)p.N : NK);
    const int tq0 = NK - NQ, qrow = tq0 + qi, base = tq0 & ~31;
    const int qs = base + (qrow - base) / (32 * R) * (32 * R);
    const int row_end = (qs + 32 * R < NK ? qs + 32 * R : NK) - 1;
    const int T = row_end / BN + 1;
    if (T == 1) return;                                    // written by its only split
    const int64_t sstride = npr;                           // (row, head) pairs per split
    const float* lse2 = p.part + (int64_t)ns * npr * D;
    float mx = -INFINITY;
    for (int sp = 0; sp < ns; ++sp) {
        if ((int64_t)T * sp / ns >= (int64_t)T * (sp + 1) / ns) continue;   // empty split
        mx = fmaxf(mx, lse2[sp * sstride + pr]);
    }
    float wsum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < ns; ++sp) {
        if ((int64_t)T * sp / ns >= (int64_t)T * (sp + 1) / ns) continue;
        const float l2 = lse2[sp * sstride + pr];
        if (l2 == -INFINITY) continue;                     // no key of this split reaches the row
        const float wgt = exp2f(l2 - mx);
        wsum += wgt;
        acc += wgt * *reinterpret_cast<const f32x4*>(p.part + (sp * sstride + pr) * D + 4 * c);
    }
    const float inv = 1.0f / wsum;
    const int64_t ob = ((row0 + qi) * p.Hq + hq) * D + 4 * c;
    if (p.out_f32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + ob) = acc * inv;
    } else {
        uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.out) + ob);
        dst[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
        dst[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    }
    if (p.lse && c == 0)
        p.lse[p.cu_q ? (row0 + qi) * p.Hq + hq : ((int64_t)b * p.Hq + hq) * NQ + qi] =
            (mx + log2f(wsum)) * 0.6931471805599453f;
}

// Compute units of the current device (cached per device).
int device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (dev >= 0 && dev < 64) n = cus[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        if (dev >= 0 && dev < 64) cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Dynamic LDS of a block-sparse launch: one bitmap of ceil(N/64) bits per compute wave (a
// workgroup takes maxw row groups of one q head) and their union, in 32-bit words.
template <int D>
size_t sparse_bitmap_bytes(int64_t N, bool haspos) {
    const size_t words = (size_t)(((N + 63) / 64 + 31) / 32);
    return (size_t)(Tile<D>::maxw(haspos) + 1) * words * 4;
}

// LDS a block-sparse launch of N tokens needs (the kernel's static arrays plus the bitmaps)
// and the device's per-workgroup limit.
template <int D, bool F32>
hipError_t sparse_lds_d(const PrefillParams& p, size_t* need, size_t* limit) {
    hipFuncAttributes attr;
    const bool hd = p.head_theta != nullptr;
    // explicit positions: the instances with a position tile
    hipError_t e = p.pos
        ? (p.counter
               ? (hd ? hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&prefill_kernel<D, F32, true, true, false, true, false, true>))
                     : hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&prefill_kernel<D, F32, true, true, false, true>)))
               : (hd ? hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&prefill_kernel<D, F32, true, false, false, true, false, true>))
                     : hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&prefill_kernel<D, F32, true, false, false, true>))))
        : p.counter
        ? (hd ? hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&prefill_kernel<D, F32, false, true, false, true, false, true>))
              : hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&prefill_kernel<D, F32, false, true, false, true>)))
        : (hd ? hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&prefill_kernel<D, F32, false, false, false, true, false, true>))
              : hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&prefill_kernel<D, F32, false, false, false, true>)));
    if (e != hipSuccess) return e;
    int dev = 0, lim = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return e;
    *need = attr.sharedSizeBytes + sparse_bitmap_bytes<D>(p.N, p.pos != nullptr);
    *limit = (size_t)lim;
    return hipSuccess;
}

// Workgroup layout of a launch: q heads per wave group, row groups per workgroup, head
// chunks, key splits.
template <int D>
Launch plan_launch(const PrefillParams& p) {
    const int G = p.Hq / p.Hkv;
    const int MAXW = Tile<D>::maxw(p.pos != nullptr);
    Launch L;
    L.ns = 1;
    if (p.blk_count) {
        // Block-sparse: a workgroup takes consecutive row groups of one q head.  Its waves'
        // lists are then one head's pattern at neighbouring query blocks, which share most
        // of their key blocks (vertical columns, nearby diagonals), so the union of tiles the
        // workgroup streams stays close to one list; grouped by heads, the union of several
        // heads' unrelated lists would approach the dense set.  (Measured on the Qwen-0.5B
        // shape: vertical-slash lists with 13% of the blocks, 0.36x the dense time against
        // 0.55x grouped by heads; random lists with 11%, 0.48x against 0.54x.)  The q heads
        // of a kv head then read the shared K/V tiles separately.
        L.nhc = G;
        L.Gc = 1;
        L.R = MAXW;
    }
    // row blocks per sequence (cached: up to 31 extra rows from aligning the first group)
    const int64_t rows = p.kv_len ? (int64_t)p.Nq + 31 : p.N;
    auto wgs = [&](int R, int nhc) { return (rows + 32 * R - 1) / (32 * R) * p.B * p.Hkv * nhc; };
    // d=128 without explicit positions: one workgroup per CU of 11 compute waves taking
    // consecutive row groups of one q head, when that still gives every CU a workgroup.
    // (Grouped by heads, 3 heads x 3 row groups = 9 waves fit: 2 SIMDs then ran 2 waves
    // instead of 3.  Measured on the Llama-3B 128K prefill: 96.2 -> 81-83 ms.  At d=64 the
    // same regrouping into one 16-wave workgroup was 9% slower than two 8-wave ones that
    // share each tile among the 7 q heads of a kv head.)
    const bool rows_grouped = p.blk_count ||
        (D == 128 && p.pos == nullptr && wgs(MAXW, G) >= (int64_t)device_cus());
    if (!p.blk_count && rows_grouped) {
        L.nhc = G;
        L.Gc = 1;
        L.R = MAXW;
    } else if (!p.blk_count) {
        const int mw = D == 128 && p.pos == nullptr ? 9 : MAXW;   // 3 x 3 at d=128
        L.nhc = (G + mw - 1) / mw;                  // head chunks, as even as possible
        L.Gc = (G + L.nhc - 1) / L.nhc;
        L.R = mw / L.Gc > 1 ? mw / L.Gc : 1;
    }
    // Cached prefill with a workspace: the key tiles of each row block shared among key
    // splits.  Asked for: exactly that many (within the workspace's room).
    const bool ksplit = p.kv_len && p.part && p.max_splits > 1;
    if (ksplit && p.splits > 0) {
        L.ns = p.splits < p.max_splits ? p.splits : p.max_splits;
        return L;
    }
    if (!rows_grouped) {
        // Few rows (a short prompt, a prefill chunk): fewer row groups per workgroup, then
        // more workgroups until about two per CU (the resident count) are launched: with a
        // workspace, by splitting each row block's key tiles (each split reads its own share
        // of the K/V tiles once, and every workgroup keeps all the q heads of its chunk);
        // without one, by spreading the q heads of a kv head over several workgroups (each
        // re-reads the kv head's K/V tiles).  (8 chunks of 4096 of the Qwen-0.5B shape: a
        // 4096-row chunk has 128 row groups per kv head, two key splits give 512 workgroups.)
        const int64_t target = 2 * (int64_t)device_cus();
        if (wgs(L.R, L.nhc) < target) {
            L.R = 1;
            const int64_t w1 = wgs(1, L.nhc);
            if (w1 < target) {
                if (ksplit) {
                    const int64_t ns = (target + w1 - 1) / w1;
                    L.ns = (int)(ns < p.max_splits ? ns : p.max_splits);
                } else {
                    int nhc = (int)((target + wgs(1, 1) - 1) / wgs(1, 1));
                    nhc = nhc < G ? nhc : G;
                    L.Gc = (G + nhc - 1) / nhc;
                    L.nhc = (G + L.Gc - 1) / L.Gc;
                }
            }
        }
    }
    return L;
}

template <int D, bool F32>
hipError_t launch_d(const PrefillParams& p, const Tables& t, hipStream_t s) {
    Launch L = plan_launch<D>(p);
    const int64_t rows = p.kv_len ? (int64_t)p.Nq + 31 : p.N;
    L.n_rb = (int)((rows + 32 * L.R - 1) / (32 * L.R));
    const int waves = L.Gc * L.R + 1;               // + the producer wave
    const int64_t nblk = (int64_t)L.n_rb * L.ns * p.B * p.Hkv * L.nhc;
    dim3 grid((unsigned)nblk), block(64 * waves);
    const bool hp = p.pos != nullptr, cn = p.counter != nullptr;
    if (p.kv_len) {
        // (per-kv-head frequency tables: the HEADS instances, windows computed per workgroup)
        const bool hd = p.head_theta != nullptr;
        if (p.pg.table) {
            if (hd && cn) prefill_kernel<D, F32, false, true, true, false, true, true><<<grid, block, 0, s>>>(p, t, L);
            else if (hd) prefill_kernel<D, F32, false, false, true, false, true, true><<<grid, block, 0, s>>>(p, t, L);
            else if (cn) prefill_kernel<D, F32, false, true, true, false, true><<<grid, block, 0, s>>>(p, t, L);
            else prefill_kernel<D, F32, false, false, true, false, true><<<grid, block, 0, s>>>(p, t, L);
        } else {
            if (hd && cn) prefill_kernel<D, F32, false, true, true, false, false, true><<<grid, block, 0, s>>>(p, t, L);
            else if (hd) prefill_kernel<D, F32, false, false, true, false, false, true><<<grid, block, 0, s>>>(p, t, L);
            else if (cn) prefill_kernel<D, F32, false, true, true, false><<<grid, block, 0, s>>>(p, t, L);
            else prefill_kernel<D, F32, false, false, true, false><<<grid, block, 0, s>>>(p, t, L);
        }
        if (L.ns > 1) {
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            const int64_t thr = (int64_t)p.B * p.Nq * p.Hq * (D / 4);
            split_combine<D><<<dim3((unsigned)((thr + 255) / 256)), dim3(256), 0, s>>>(p, L.R, L.ns);
        }
    } else if (p.blk_count) {
        // block bitmaps: one per compute wave and their union (the caller has checked that
        // they fit next to the kernel's static LDS: sparse_lds)
        const size_t bits = sparse_bitmap_bytes<D>(p.N, hp);
        const bool hd = p.head_theta != nullptr;        // per-kv-head frequency tables
        // explicit positions: blocks stay token-index blocks, distances come from the
        // position tile
        if (hp && hd && cn) prefill_kernel<D, F32, true, true, false, true, false, true><<<grid, block, bits, s>>>(p, t, L);
        else if (hp && hd) prefill_kernel<D, F32, true, false, false, true, false, true><<<grid, block, bits, s>>>(p, t, L);
        else if (hp && cn) prefill_kernel<D, F32, true, true, false, true><<<grid, block, bits, s>>>(p, t, L);
        else if (hp) prefill_kernel<D, F32, true, false, false, true><<<grid, block, bits, s>>>(p, t, L);
        else if (hd && cn) prefill_kernel<D, F32, false, true, false, true, false, true><<<grid, block, bits, s>>>(p, t, L);
        else if (hd) prefill_kernel<D, F32, false, false, false, true, false, true><<<grid, block, bits, s>>>(p, t, L);
        else if (cn) prefill_kernel<D, F32, false, true, false, true><<<grid, block, bits, s>>>(p, t, L);
        else prefill_kernel<D, F32, false, false, false, true><<<grid, block, bits, s>>>(p, t, L);
    } else if (p.head_theta) {
        // per-head rotation frequencies (one-shot prefill only)
        if (hp && cn) prefill_kernel<D, F32, true, true, false, false, false, true><<<grid, block, 0, s>>>(p, t, L);
        else if (hp) prefill_kernel<D, F32, true, false, false, false, false, true><<<grid, block, 0, s>>>(p, t, L);
        else if (cn) prefill_kernel<D, F32, false, true, false, false, false, true><<<grid, block, 0, s>>>(p, t, L);
        else prefill_kernel<D, F32, false, false, false, false, false, true><<<grid, block, 0, s>>>(p, t, L);
    } else if (hp && cn) prefill_kernel<D, F32, true, true, false, false><<<grid, block, 0, s>>>(p, t, L);
    else if (hp) prefill_kernel<D, F32, true, false, false, false><<<grid, block, 0, s>>>(p, t, L);
    else if (cn) prefill_kernel<D, F32, false, true, false, false><<<grid, block, 0, s>>>(p, t, L);
    else prefill_kernel<D, F32, false, false, false, false><<<grid, block, 0, s>>>(p, t, L);
    return hipGetLastError();
}

}  // namespace

hipError_t prefill_sparse_lds(const PrefillParams& p, size_t* need, size_t* limit) {
    if (p.d == 64) return p.in_f32 ? sparse_lds_d<64, true>(p, need, limit) : sparse_lds_d<64, false>(p, need, limit);
    return p.in_f32 ? sparse_lds_d<128, true>(p, need, limit) : sparse_lds_d<128, false>(p, need, limit);
}

int prefill_key_splits(const PrefillParams& p) {
    return p.d == 64 ? plan_launch<64>(p).ns : plan_launch<128>(p).ns;
}

hipError_t launch_prefill(const PrefillParams& p, const Tables& t, hipStream_t s) {
    if (!p.kv_len && (p.Np % Tile<64>::BN || p.Np % Tile<128>::BN)) return hipErrorInvalidValue;
    if (p.d == 64) return p.in_f32 ? launch_d<64, true>(p, t, s) : launch_d<64, false>(p, t, s);
    return p.in_f32 ? launch_d<128, true>(p, t, s) : launch_d<128, false>(p, t, s);
}

}  // namespace wpa

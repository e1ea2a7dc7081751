// Key rotation and K/V relayout.
//
// (A decode cache may keep a pair block only for the keys still inside that block's
// largest window: such a block is a ring over tokens, see KLayout.)
//
// Keys are rotated once, at their own position (ATFlash abstract: the RoPE score is a
// sum over 2-D rotation pairs), and stored pair-blocked: block j of a head holds pairs
// 8j..8j+7, as the 8 first-half components followed by the 8 second-half components,
// [B][Hkv][d/16][tokens][16] in IEEE half precision (the rotated value of a bf16 input
// needs more than bf16's 8 significant bits; half keeps 11, at the same MFMA rate, for
// rotated components below 65504 in magnitude).  One 16-element block is one MFMA K-step, so
// contracting only the active blocks (pairs form a contiguous slice of the contraction
// axis at every distance) reads contiguous memory for every token range.
//
// Values, for prefill and for the decode cache alike, are blocked by key octets,
// [B][Hkv][tokens/8][d][8]: the P*V matrix product (a contraction over keys) then reads
// key-contiguous 16-byte MFMA operands, and a tile of keys is one contiguous block.
#include "wpa_device.hpp"
#include "wpa_internal.hpp"

namespace wpa {

// Thread id of the key rotation: one (sequence, kv head, pair block, token).
template <bool F32>
__device__ inline void rope_keys_item(const RopeParams& p, const Tables& tab, int64_t id) {
    const int NB = p.d / 16;
    const int P = p.d / 2;
    const int64_t ntok = p.pad_to > p.n ? p.pad_to : p.n;
    const int64_t total = (int64_t)p.B * p.Hkv * NB * ntok;
    if (id >= total) return;
    const int64_t t = id % ntok;
    int64_t rest = id / ntok;
    const int j = (int)(rest % NB);
    rest /= NB;
    const int g = (int)(rest % p.Hkv);
    const int b = (int)(rest / p.Hkv);

    // block j's rows (layout kl); a ring block takes token tok in row tok mod cap, and only
    // the newest cap tokens of this write (an older one would share a row with a newer)
    int64_t off = p.kl.off[0];
    int cap = p.kl.cap[0];
#pragma unroll
    for (int jj = 1; jj < 8; ++jj)
        if (j == jj) {
            off = p.kl.off[jj];
            cap = p.kl.cap[jj];
        }
    const int64_t tok = p.t0 + t;
    uint16_t* dst;
    if (p.pg.table) {
        // paged: row tok mod page of block j of the page holding tok
        const int64_t page = page_of(p.pg, b, tok);
        const int64_t ps = (int64_t)1 << p.pg.page_log2;
        dst = p.kp + (((page * p.Hkv + g) * NB + j) * ps + (tok & (ps - 1))) * 16;
    } else {
        int64_t krow = tok;
        if (cap < p.ld) {
            if (tok + cap < p.t0 + p.n) return;
            krow = tok % cap;
        }
        dst = p.kp + (((int64_t)b * p.Hkv + g) * p.kl.head + off + krow) * 16;
    }
    u32x4* d4 = reinterpret_cast<u32x4*>(dst);
    if (t >= p.n) {
        u32x4 z = {0u, 0u, 0u, 0u};
        d4[0] = z;
        d4[1] = z;
        return;
    }
    const int64_t row = (((int64_t)b * p.n + t) * p.Hkv + g) * p.d;
    float x[8], y[8];
    if (p.interleaved) {
        // pairs 8j..8j+7 are dims 16j..16j+15, each pair's two components adjacent
        float a[8], c[8];
        load8<F32>(p.k, row + 16 * j, a);
        load8<F32>(p.k, row + 16 * j + 8, c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = a[2 * e];
            y[e] = a[2 * e + 1];
            x[4 + e] = c[2 * e];
            y[4 + e] = c[2 * e + 1];
        }
    } else {
        load8<F32>(p.k, row + 8 * j, x);
        load8<F32>(p.k, row + P + 8 * j, y);
    }
    const int64_t pos = p.pos ? (int64_t)p.pos[(int64_t)b * p.n + t] : p.t0 + t;
    // rotation frequencies: the shared table, or kv head g's row of the per-head tables
    const double* hth = p.head_theta ? p.head_theta + (int64_t)g * P : nullptr;
    auto TH = [&](int i) { return hth ? hth[i] : tab.theta[i]; };
    uint32_t ox[4], oy[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        float s0, c0, s1, c1;
        rope_sincos(pos, TH(8 * j + e), &s0, &c0);
        rope_sincos(pos, TH(8 * j + e + 1), &s1, &c1);
        float x0 = round_bf16(x[e]), y0 = round_bf16(y[e]);
        float x1 = round_bf16(x[e + 1]), y1 = round_bf16(y[e + 1]);
        ox[e / 2] = pack_f16x2(x0 * c0 - y0 * s0, x1 * c1 - y1 * s1);
        oy[e / 2] = pack_f16x2(y0 * c0 + x0 * s0, y1 * c1 + x1 * s1);
    }
    d4[0] = u32x4{ox[0], ox[1], ox[2], ox[3]};
    d4[1] = u32x4{oy[0], oy[1], oy[2], oy[3]};
}

template <bool F32>
__global__ __launch_bounds__(256) void rope_keys_kernel(RopeParams p, Tables tab) {
    rope_keys_item<F32>(p, tab, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// V for prefill, by key octets [B][Hkv][ntok/8][d][8] bf16, zero past the last token:
// one block = 64 tokens (8 octets) x d dims of one (b, kv head), staged through LDS so that
// both the token-row reads and the octet writes are contiguous.
template <bool F32, int D>
__global__ __launch_bounds__(256) void v_octets_kernel(RopeParams p) {
    __shared__ uint16_t tile[64][D + 2];
    const int64_t ntok = p.pad_to > p.n ? p.pad_to : p.n;
    const int64_t ntiles = (ntok + 63) / 64;
    const int64_t tile_id = blockIdx.x % ntiles;
    const int bg = blockIdx.x / ntiles;
    const int g = bg % p.Hkv, b = bg / p.Hkv;
    const int64_t t0 = tile_id * 64;
    // load: each thread 8 elements of one token row
    for (int c = threadIdx.x; c < 64 * (D / 8); c += blockDim.x) {
        const int tt = c / (D / 8), e8 = (c % (D / 8)) * 8;
        const int64_t t = t0 + tt;
        float x[8];
        if (t < p.n) {
            load8<F32>(p.v, (((int64_t)b * p.n + t) * p.Hkv + g) * D + e8, x);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) tile[tt][e8 + i] = f32_to_bf16_bits(x[i]);
    }
    __syncthreads();
    // store: each thread the 8 tokens of one octet for one dim; consecutive threads write
    // consecutive 16-byte pieces (dims of one octet, then the next octet)
    for (int c = threadIdx.x; c < D * 8; c += blockDim.x) {
        const int oc = c / D, e = c % D, t8 = 8 * oc;
        const int64_t t = t0 + t8;
        if (t >= ntok) continue;
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = (uint32_t)tile[t8 + 2 * i][e] | ((uint32_t)tile[t8 + 2 * i + 1][e] << 16);
        uint16_t* dst = p.vout + ((((int64_t)b * p.Hkv + g) * (p.ld / 8) + (p.t0 + t) / 8) * D + e) * 8;
        *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
    }
}

// V into the decode cache, key-octet blocked: [B][Hkv][ceil(Lmax/8)][d][8] bf16, i.e. for
// every 8 consecutive tokens each dim's 8 values are contiguous (16 bytes).  That is the
// operand layout of the P*V matrix product in decode (contraction over keys).  One thread
// handles one (sequence, kv head, octet, 8 dims): an 8x8 transpose in registers; tokens of a
// partially written octet keep their previous cache contents.
template <bool F32>
__device__ inline void v_cache_item(const RopeParams& p, int64_t id) {
    const int d8 = p.d / 8;
    const int64_t o_first = p.t0 / 8, o_last = (p.t0 + p.n - 1) / 8;
    const int64_t n_oct = o_last - o_first + 1;
    const int64_t total = (int64_t)p.B * p.Hkv * n_oct * d8;
    if (id >= total) return;
    const int e8 = (int)(id % d8) * 8;
    int64_t rest = id / d8;
    const int64_t o = o_first + rest % n_oct;
    rest /= n_oct;
    const int g = (int)(rest % p.Hkv);
    const int b = (int)(rest / p.Hkv);
    uint16_t* dst;
    if (p.pg.table) {
        // paged: octet (8o mod page)/8 of the page holding token 8o
        const int64_t page = page_of(p.pg, b, 8 * o);
        const int64_t o_pg = (int64_t)1 << (p.pg.page_log2 - 3);        // octets per page
        dst = p.vout + (((page * p.Hkv + g) * o_pg + (o & (o_pg - 1))) * p.d + e8) * 8;
    } else {
        const int64_t L8 = (p.ld + 7) / 8;
        dst = p.vout + ((((int64_t)b * p.Hkv + g) * L8 + o) * p.d + e8) * 8;
    }
    uint16_t cell[8][8];                 // [dim][token in octet]
    const bool partial = o * 8 < p.t0 || o * 8 + 8 > p.t0 + p.n;
    if (partial) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const u32x4 w = reinterpret_cast<const u32x4*>(dst)[e];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                cell[e][2 * i] = (uint16_t)(w[i] & 0xffffu);
                cell[e][2 * i + 1] = (uint16_t)(w[i] >> 16);
            }
        }
    }
#pragma unroll
    for (int t8 = 0; t8 < 8; ++t8) {
        const int64_t t = o * 8 + t8 - p.t0;            // source row
        if (t < 0 || t >= p.n) continue;
        float x[8];
        load8<F32>(p.v, (((int64_t)b * p.n + t) * p.Hkv + g) * p.d + e8, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) cell[e][t8] = f32_to_bf16_bits(x[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = (uint32_t)cell[e][2 * i] | ((uint32_t)cell[e][2 * i + 1] << 16);
        reinterpret_cast<u32x4*>(dst)[e] = w;
    }
}

// A cache append in one launch: the first k_blocks workgroups rotate keys, the rest write V
// (one launch instead of two: the appends of a chunked prefill are small, so the second
// launch was about half of their cost).
template <bool F32>
__global__ __launch_bounds__(256) void kv_cache_kernel(RopeParams p, Tables tab, unsigned k_blocks) {
    if (blockIdx.x < k_blocks) rope_keys_item<F32>(p, tab, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
    else v_cache_item<F32>(p, (int64_t)(blockIdx.x - k_blocks) * blockDim.x + threadIdx.x);
}

hipError_t launch_rope_relayout(const RopeParams& p, hipStream_t s) {
    const int NB = p.d / 16;
    const int64_t ntok = p.pad_to > p.n ? p.pad_to : p.n;
    const int64_t nk = (int64_t)p.B * p.Hkv * NB * ntok;
    dim3 blk(256);
    const unsigned kb = (unsigned)((nk + 255) / 256);
    if (!p.v_prefill) {
        const int64_t n_oct = (p.t0 + p.n - 1) / 8 - p.t0 / 8 + 1;
        const int64_t nv = (int64_t)p.B * p.Hkv * n_oct * (p.d / 8);
        dim3 grid(kb + (unsigned)((nv + 255) / 256));
        if (p.in_f32) kv_cache_kernel<true><<<grid, blk, 0, s>>>(p, *p.tab, kb);
        else kv_cache_kernel<false><<<grid, blk, 0, s>>>(p, *p.tab, kb);
        return hipGetLastError();
    }
    if (p.in_f32)
        rope_keys_kernel<true><<<dim3(kb), blk, 0, s>>>(p, *p.tab);
    else
        rope_keys_kernel<false><<<dim3(kb), blk, 0, s>>>(p, *p.tab);
    {
        const int64_t nt = (ntok + 63) / 64;
        dim3 grid((unsigned)(nt * p.B * p.Hkv));
        if (p.d == 64) {
            if (p.in_f32) v_octets_kernel<true, 64><<<grid, blk, 0, s>>>(p);
            else v_octets_kernel<false, 64><<<grid, blk, 0, s>>>(p);
        } else {
            if (p.in_f32) v_octets_kernel<true, 128><<<grid, blk, 0, s>>>(p);
            else v_octets_kernel<false, 128><<<grid, blk, 0, s>>>(p);
        }
    }
    return hipGetLastError();
}

}  // namespace wpa

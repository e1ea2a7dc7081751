// One decode step with the per-RoPE-wavelength window (ATFlash abstract: the window
// ported into a decode kernel), split over the KV sequence, on MFMA (q.k in half
// precision, P*V in bf16).
//
// Work item = (sequence b, kv head g, chunk of `chunk` keys); items past kv_len exit.
// Each item serves all G q heads of its kv head, so every K/V byte is read once per step.
// The 4 waves take interleaved 32-key tiles of the chunk, each with its own online-softmax
// state, merged in LDS at the end.
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
#include "wpa_device.hpp"
#include "wpa_internal.hpp"

namespace wpa {

namespace {

constexpr int kWaves = 4;
constexpr float kTau = 8.0f;

__device__ inline int perm_row(int m) {
    return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ inline float xchg32(float v, int xaddr) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(xaddr, __builtin_bit_cast(int, v)));
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void decode_partial_kernel(DecodeParams p, Tables tab) {
    constexpr int NB = D / 16;
    constexpr int P = D / 2;
    constexpr int NDB = D / 32;
    constexpr int GMAX = 16;                        // q heads per kv head (columns used)
    __shared__ __attribute__((aligned(16))) uint16_t sQ[32][D];      // pair-blocked, half
    __shared__ float sO[kWaves][GMAX][D + 2];

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
    const int xaddr = (lane ^ 32) << 2;
    const int G = p.Hq / p.Hkv;
    const int chunk = blockIdx.x % p.n_chunks;
    const int bg = blockIdx.x / p.n_chunks;
    const int g = bg % p.Hkv, b = bg / p.Hkv;
    const int Lb = __builtin_amdgcn_readfirstlane(p.kv_len[b]);
    const int c0 = chunk * p.chunk;
    if (c0 >= Lb) return;
    const int c1 = c0 + p.chunk < Lb ? c0 + p.chunk : Lb;
    const int64_t qpos = __builtin_amdgcn_readfirstlane(p.q_pos ? p.q_pos[b] : Lb - 1);
    const float sl2 = p.scale * 1.4426950408889634f;

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
            rope_sincos(qpos, tab.theta[pr], &sn, &cs);
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

    const uint16_t* kpg = p.kp + ((int64_t)b * p.Hkv + g) * p.kl.head * 16;
    const int64_t L8 = (p.Lmax + 7) / 8;
    const uint16_t* vg = p.v + ((int64_t)b * p.Hkv + g) * L8 * D * 8;

    f32x16 O[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) O[i] = f32x16{};
    float m = -INFINITY, lsum = 0.f;
    uint64_t cnt = 0;
    const int arow = perm_row(l32);                  // key row this lane feeds to the A operand

    const char* kbytes = reinterpret_cast<const char*>(kpg);
    const char* vbytes = reinterpret_cast<const char*>(vg);
    const uint32_t voff0 = (uint32_t)((h * D + l32) * 16);
    int plo = 0, pfull = 0;                          // band edges, moved incrementally
    for (int k0 = c0 + 32 * w; k0 < c1; k0 += 32 * kWaves) {
        const int kmax = k0 + 31 < c1 ? k0 + 31 : c1 - 1;
        int64_t dlo, dhi;
        if (qpos >= kmax) { dlo = qpos - kmax; dhi = qpos - k0; }
        else if (qpos <= k0) { dlo = k0 - qpos; dhi = kmax - qpos; }
        else { dlo = 0; dhi = (qpos - k0 > kmax - qpos) ? qpos - k0 : kmax - qpos; }
        const int dl = __builtin_amdgcn_readfirstlane((int)(dlo < INT32_MAX ? dlo : INT32_MAX));
        const int dh = __builtin_amdgcn_readfirstlane((int)(dhi < INT32_MAX ? dhi : INT32_MAX));
        // first pair with W >= dl (resp. dh); consecutive tiles of a wave move these by a
        // step or two, so walk from the previous value instead of searching
        while (plo > 0 && tab.W[plo - 1] >= dl) --plo;
        while (plo < P && tab.W[plo] < dl) ++plo;
        while (pfull > 0 && tab.W[pfull - 1] >= dh) --pfull;
        while (pfull < P && tab.W[pfull] < dh) ++pfull;
        plo = __builtin_amdgcn_readfirstlane(plo);
        pfull = __builtin_amdgcn_readfirstlane(pfull);
        const int jlo = plo >> 3;
        const bool tail = k0 + 32 > c1;             // tile runs past the chunk's last key

        // issue every load of the tile before using any: active K blocks (lane = key row
        // arow, half h) and the V^T operands (lane = dim, half h = key octet); uniform
        // 64-bit bases with 32-bit lane offsets.  The caches are streamed once per step:
        // non-temporal loads (a plain read runs markedly closer to the HBM peak with them)
        const int key = k0 + arow;
        const int keyc = key < c1 ? key : c1 - 1;
        u32x4 ka[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            if (j < jlo) continue;
            // row of this key in block j: the key itself, or in a ring block (one holding only
            // the keys inside its largest window) key mod cap, without wrapping in the tile
            const int cap = p.kl.cap[j];
            const int r0 = cap < p.Lmax ? (int)((uint32_t)k0 % (uint32_t)cap) : k0;
            const int64_t koff = (p.kl.off[j] + r0) * 32 + (int64_t)((keyc - k0) * 32 + 16 * h);
            ka[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbytes + koff));
        }
        u32x4 va[2][NDB];
        const int64_t oct0 = k0 >> 3;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            // octet oct0 + 2c + h; the last octet of the cache stands in past its end
            const int64_t ob = oct0 + 2 * c + 1 < L8 ? oct0 + 2 * c : L8 - 1 - h;
            const char* vb = vbytes + ob * (D * 16);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                va[c][db] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + voff0 + db * 512));
        }

        // S^T over the active blocks; pairs not active for this lane's key are zeroed
        const int64_t dist = qpos - key >= 0 ? qpos - key : key - qpos;
        f32x16 S = f32x16{};
#pragma unroll
        for (int j = NB - 1; j >= 0; --j) {
            if (j < jlo) continue;
            u32x4 a = ka[j];
            int on = 8;
            if (8 * j < pfull) {                      // block holds a straddling pair
                on = 0;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const bool e0 = dist <= (int64_t)tab.W[8 * j + 2 * t];
                    const bool e1 = dist <= (int64_t)tab.W[8 * j + 2 * t + 1];
                    on += e0 + e1;
                    a[t] &= (e0 ? 0xffffu : 0u) | (e1 ? 0xffff0000u : 0u);
                }
            }
            if (p.counter && h == 0 && key < c1) cnt += on;
            S = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, qB[j]), S,
                                                       0, 0, 0);
        }

        // register r of half h holds key k0 + 16(r/8) + 8h + (r%8) for column l32
        if (tail) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (k0 + 16 * (r >> 3) + 8 * h + (r & 7) >= c1) S[r] = -INFINITY;
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
                        a[t] &= (kb + 2 * t < c1 ? 0xffffu : 0u) | (kb + 2 * t + 1 < c1 ? 0xffff0000u : 0u);
                }
                O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, pb), O[db], 0, 0, 0);
            }
        }
    }

    if (p.counter) {
        uint64_t tot = cnt;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o);
        if (lane == 0 && tot) atomicAdd(p.counter, (unsigned long long)(tot * (uint64_t)G));
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
}

// out[b][hq] = merge over the chunks c < ceil(kv_len/chunk) of the partials.
// Block = 256 threads = 8 chunk groups x 32 dims; grid = (B*Hq) x (D/32).
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p) {
    __shared__ float red[256];
    __shared__ float sacc[8][33];
    const int tid = threadIdx.x;
    const int bh = blockIdx.x, slice = blockIdx.y;
    const int b = bh / p.Hq, hq = bh % p.Hq;
    const int G = p.Hq / p.Hkv;
    const int g = hq / G, hh = hq % G;
    const int64_t Lb = __builtin_amdgcn_readfirstlane(p.kv_len[b]);
    const int nc = (int)((Lb + p.chunk - 1) / p.chunk);
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
    decode_partial_kernel<D><<<grid, block, 0, s>>>(p, t);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid2((unsigned)(p.B * p.Hq), D / 32), block2(256);
    decode_combine_kernel<D><<<grid2, block2, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, const Tables& t, hipStream_t s) {
    return p.d == 64 ? launch_decode_d<64>(p, t, s) : launch_decode_d<128>(p, t, s);
}

}  // namespace wpa

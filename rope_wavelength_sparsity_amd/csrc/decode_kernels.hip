// One decode step with the per-RoPE-wavelength window (ATFlash abstract: the window
// ported into a decode kernel), split over the KV sequence.
//
// Work item = (sequence b, kv head g, chunk of `chunk` keys); items past kv_len exit.
// Each item serves all G q heads of its kv head, so every K/V byte is read once per step.
//
// The keys of a wave (64 consecutive cache entries, lane = key) span a distance band
// [dlo, dhi]; pairs with W_i < dlo are inactive for all of them, so the 16-dim blocks
// below the first pair with W_i >= dlo are never read: far keys load only the blocks of
// the long-wavelength pairs still inside their window (the K cache is pair-blocked, so
// each block of 64 keys is one contiguous 2 KB run).  Blocks holding a pair whose
// threshold falls inside the band are masked per key and pair; the test is D <= W_i.
//
// QK: VALU dot products, lane = key, q' broadcast from LDS.  Softmax: wavefront max
// reductions, exp2 domain, lazy rescale (exact).  P*V: lane = (key group, 8-dim group),
// coalesced 16-byte V loads.  Partials (O, m, l) per (item, q head) are merged in LDS
// across the 4 waves and written out; the combine kernel merges chunks.
#include "wpa_device.hpp"
#include "wpa_internal.hpp"

namespace wpa {

namespace {

constexpr int kWaves = 4;
constexpr float kTau = 8.0f;

template <int D, int GM>
__global__ __launch_bounds__(256) void decode_partial_kernel(DecodeParams p, Tables tab) {
    constexpr int NB = D / 16;
    constexpr int P = D / 2;
    constexpr int LPK = D / 8;            // lanes per key row in the P*V phase
    constexpr int KPL = 64 / LPK;         // keys per wave-wide V load
    __shared__ __attribute__((aligned(16))) float sQ[GM][D];
    __shared__ float sP[kWaves][GM][64];
    __shared__ float sM[kWaves][GM], sL[kWaves][GM];
    __shared__ __attribute__((aligned(16))) float sO[kWaves][GM][D];

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int G = p.Hq / p.Hkv;
    const int chunk = blockIdx.x % p.n_chunks;
    const int bg = blockIdx.x / p.n_chunks;
    const int g = bg % p.Hkv, b = bg / p.Hkv;
    const int64_t Lb = p.kv_len[b];
    const int64_t c0 = (int64_t)chunk * p.chunk;
    if (c0 >= Lb) return;
    const int64_t c1 = c0 + p.chunk < Lb ? c0 + p.chunk : Lb;
    const int64_t qpos = p.q_pos ? (int64_t)p.q_pos[b] : Lb - 1;

    // rotate the G query heads of this kv head into pair-blocked fp32 in LDS
    for (int i = tid; i < GM * P; i += blockDim.x) {
        const int hh = i / P, pr = i % P;
        if (hh >= G) continue;
        const int64_t qb = ((int64_t)b * p.Hq + g * G + hh) * D;
        float x, y;
        if (p.in_f32) {
            x = round_bf16(static_cast<const float*>(p.q)[qb + pr]);
            y = round_bf16(static_cast<const float*>(p.q)[qb + P + pr]);
        } else {
            x = bf16_bits_to_f32(static_cast<const uint16_t*>(p.q)[qb + pr]);
            y = bf16_bits_to_f32(static_cast<const uint16_t*>(p.q)[qb + P + pr]);
        }
        float s, c;
        rope_sincos(qpos, tab.theta[pr], &s, &c);
        const int j = pr >> 3, e = pr & 7;
        sQ[hh][16 * j + e] = round_bf16(x * c - y * s);
        sQ[hh][16 * j + 8 + e] = round_bf16(y * c + x * s);
    }
    __syncthreads();

    const uint16_t* kpg = p.kp + ((int64_t)b * p.Hkv + g) * NB * p.Lmax * 16;
    const uint16_t* vg = p.v + ((int64_t)b * p.Hkv + g) * p.Lmax * D;
    const float sl2 = p.scale * 1.4426950408889634f;
    const int kg = lane / LPK, dg = lane % LPK;

    float m[GM], l[GM], acc[GM][8];
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
        m[hh] = -INFINITY;
        l[hh] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[hh][i] = 0.f;
    }
    uint64_t cnt = 0;

    for (int64_t kw0 = c0 + 64 * w; kw0 < c1; kw0 += 64 * kWaves) {
        const int64_t key = kw0 + lane;
        const bool kvalid = key < c1;
        const int64_t kmax = (kw0 + 63 < c1 ? kw0 + 63 : c1 - 1);
        const int64_t dist = qpos - key >= 0 ? qpos - key : key - qpos;
        int64_t dlo, dhi;
        if (qpos >= kmax) { dlo = qpos - kmax; dhi = qpos - kw0; }
        else if (qpos <= kw0) { dlo = kw0 - qpos; dhi = kmax - qpos; }
        else { dlo = 0; dhi = (qpos - kw0 > kmax - qpos) ? qpos - kw0 : kmax - qpos; }
        const int plo = first_at_least(tab.W, P, dlo);
        const int pfull = first_at_least(tab.W, P, dhi);

        float s[GM];
#pragma unroll
        for (int hh = 0; hh < GM; ++hh) s[hh] = 0.f;
        for (int j = plo >> 3; j < NB; ++j) {
            u32x4 wx = {0u, 0u, 0u, 0u}, wy = {0u, 0u, 0u, 0u};
            if (kvalid) {
                const u32x4* src = reinterpret_cast<const u32x4*>(kpg + ((int64_t)j * p.Lmax + key) * 16);
                wx = src[0];
                wy = src[1];
            }
            float kx[8], ky[8];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                kx[2 * t] = bf16_bits_to_f32(wx[t] & 0xffffu);
                kx[2 * t + 1] = bf16_bits_to_f32(wx[t] >> 16);
                ky[2 * t] = bf16_bits_to_f32(wy[t] & 0xffffu);
                ky[2 * t + 1] = bf16_bits_to_f32(wy[t] >> 16);
            }
            if (8 * j < pfull) {       // block holds a pair not active for every key
                int on_count = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bool on = dist <= (int64_t)tab.W[8 * j + e];
                    on_count += on;
                    kx[e] = on ? kx[e] : 0.f;
                    ky[e] = on ? ky[e] : 0.f;
                }
                if (kvalid) cnt += on_count;
            } else if (kvalid) {
                cnt += 8;
            }
#pragma unroll
            for (int hh = 0; hh < GM; ++hh) {
                if (hh >= G) continue;
                const f32x4* qx = reinterpret_cast<const f32x4*>(&sQ[hh][16 * j]);
                const f32x4 a0 = qx[0], a1 = qx[1], b0 = qx[2], b1 = qx[3];
                float t = s[hh];
                t += a0[0] * kx[0] + a0[1] * kx[1] + a0[2] * kx[2] + a0[3] * kx[3];
                t += a1[0] * kx[4] + a1[1] * kx[5] + a1[2] * kx[6] + a1[3] * kx[7];
                t += b0[0] * ky[0] + b0[1] * ky[1] + b0[2] * ky[2] + b0[3] * ky[3];
                t += b1[0] * ky[4] + b1[1] * ky[5] + b1[2] * ky[6] + b1[3] * ky[7];
                s[hh] = t;
            }
        }

#pragma unroll
        for (int hh = 0; hh < GM; ++hh) {
            if (hh >= G) continue;
            const float t = kvalid ? s[hh] * sl2 : -INFINITY;
            const float mx = wave_max(t);
            const float m_new = fmaxf(m[hh], mx);
            if (m_new > m[hh] + kTau) {          // uniform: m and mx are wave-wide
                const float alpha = exp2f(m[hh] - m_new);
                l[hh] *= alpha;
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[hh][i] *= alpha;
                m[hh] = m_new;
            }
            const float pr = exp2f(t - m[hh]);
            l[hh] += pr;
            sP[w][hh][lane] = pr;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0): own LDS writes done
        __builtin_amdgcn_wave_barrier();

        // P*V: lane = (key group kg, dims 8*dg .. 8*dg+7)
#pragma unroll 4
        for (int it = 0; it < 64 / KPL; ++it) {
            const int kl = it * KPL + kg;
            const int64_t kk = kw0 + kl;
            if (kk >= c1) continue;
            float vv[8];
            load8<false>(vg, kk * D + 8 * dg, vv);
#pragma unroll
            for (int hh = 0; hh < GM; ++hh) {
                if (hh >= G) continue;
                const float pw = sP[w][hh][kl];
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[hh][i] += pw * vv[i];
            }
        }
        __builtin_amdgcn_wave_barrier();
    }

    // merge the key groups of this wave (same dims, same running max)
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
        if (hh >= G) continue;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float v = acc[hh][i];
#pragma unroll
            for (int o = LPK; o < 64; o <<= 1) v += __shfl_xor(v, o);
            acc[hh][i] = v;
        }
        const float lw = wave_sum(l[hh]);
        if (lane < LPK) {
#pragma unroll
            for (int i = 0; i < 8; ++i) sO[w][hh][8 * lane + i] = acc[hh][i];
        }
        if (lane == 0) {
            sM[w][hh] = m[hh];
            sL[w][hh] = lw;
        }
    }
    if (p.counter) {
        uint64_t tot = cnt;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o);
        if (lane == 0 && tot) atomicAdd(p.counter, (unsigned long long)(tot * (uint64_t)G));
    }
    __syncthreads();

    // merge the 4 waves and write this item's partial (O relative to M, M, l)
    float* dst = p.partial + ((int64_t)bg * p.n_chunks + chunk) * G * (D + 2);
    for (int i = tid; i < G * D; i += blockDim.x) {
        const int hh = i / D, e = i % D;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sM[ww][hh]);
        float o = 0.f, ls = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float f = exp2f(sM[ww][hh] - M);
            o += f * sO[ww][hh][e];
            ls += f * sL[ww][hh];
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
    const int64_t Lb = p.kv_len[b];
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

template <int D, int GM>
void launch_partial(const DecodeParams& p, const Tables& t, hipStream_t s) {
    dim3 grid((unsigned)((int64_t)p.n_chunks * p.B * p.Hkv)), block(64 * kWaves);
    decode_partial_kernel<D, GM><<<grid, block, 0, s>>>(p, t);
}

template <int D>
hipError_t launch_decode_d(const DecodeParams& p, const Tables& t, hipStream_t s) {
    const int G = p.Hq / p.Hkv;
    if (G <= 1) launch_partial<D, 1>(p, t, s);
    else if (G <= 2) launch_partial<D, 2>(p, t, s);
    else if (G <= 4) launch_partial<D, 4>(p, t, s);
    else if (G <= 8) launch_partial<D, 8>(p, t, s);
    else launch_partial<D, 16>(p, t, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)(p.B * p.Hq), D / 32), block(256);
    decode_combine_kernel<D><<<grid, block, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, const Tables& t, hipStream_t s) {
    return p.d == 64 ? launch_decode_d<64>(p, t, s) : launch_decode_d<128>(p, t, s);
}

}  // namespace wpa

// Backward of the causal prefill with a per-RoPE-wavelength window, on gfx950 MFMA
// (WavePrune, What the paper found: models trained with the window need its gradients).
//
// For dout = dL/dout, with P the windowed softmax of the forward (recomputed from the
// forward's lse), per q head and per visible (row r, key c):
//   dP_rc = dout_r . v_c,   D_r = dout_r . out_r,   dl_rc = P_rc (dP_rc - D_r)
//   dv_c  = sum_r P_rc dout_r
//   dq'_r = scale * sum_c dl_rc [pair of x kept at r-c] k'_c[x]    (rotated coordinates)
//   dk'_c = scale * sum_r dl_rc [pair of x kept at r-c] q'_r[x]
// and dq, dk are dq', dk' rotated back by minus the RoPE angle.  The window keeps a pair's
// term only inside its distance, so in the dq and dk contractions each 32x32 block uses the
// same band plan as the forward: dims of dead pairs are skipped, fully active pairs are one
// MFMA per 16-dim block, and each pair whose window edge falls inside the block is one MFMA
// with dl masked to the elements inside its window.
//
// Kernels
//   bwd_prep_k: rotated keys, pair-blocked K' [B][Hkv][d/16][Np][16] and K'^T by key octets
//               [B][Hkv][Np/8][d][8] (pair-block element order), IEEE half; V blocked by 16
//               dims [B][Hkv][d/16][Np][16] bf16.
//   bwd_prep_q: rotated queries Q' (times scale*log2 e) pair-blocked, Q'^T (unscaled) by row
//               octets, dout blocked by 16 dims and by row octets (bf16), lse*log2 e and D
//               per row.
//   bwd_dq:     a workgroup per (sequence, kv head, row block): each compute wave takes one q
//               head's 32 query rows; S^T, P^T, dP^T, dl^T over the causal key tiles streamed
//               through LDS, dq'^T on MFMA; epilogue rotates back and writes dq.
//   bwd_dkdv:   a workgroup per (sequence, q head, key block): each compute wave takes 32
//               keys; S, P, dP, dl over the causal row tiles streamed through LDS, dv^T and
//               dk'^T on MFMA, written per q head to a workspace (d = 128: a dv pass and a
//               dk pass, each with half the accumulators and more waves).
//   bwd_reduce: sums the q heads of each kv head, rotates dk' back, writes dk and dv.
// Workgroups are ordered longest ranges first (dq: the last row blocks; dk, dv: the first
// key blocks), so that short ones fill the tail.
//
// MFMA layouts (32x32x16): A row m / B column n in lane m%32 / n%32, the 16-deep contraction
// split 8+8 between lane halves; C element (8(r/4) + 4(l/32) + r%4, l%32) in register r of
// lane l.  A-operand rows are permuted (bits 2 and 3 swapped) wherever the result feeds a
// contraction over that index, so that C registers 0-7 / 8-15 of lane half h hold indices
// 8h..8h+7 / 16+8h..16+8h+7: exactly the B operand of the next MFMA.
#include "wpa_device.hpp"
#include "wpa_internal.hpp"

namespace wpa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((address_space(3))) void* lds_ptr;

// Workgroup layout of the dq kernel: q heads per wave group, row groups per workgroup, head
// chunks per kv head, row blocks per sequence.
struct BwdLaunch {
    int Gc, R, nhc, n_rb;
};

__device__ inline int perm_row(int m) {
    return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Index (row or key) held by C register r of lane half h when the A rows were permuted.
__device__ inline int idx_of_reg(int r, int h) {
    return 16 * (r >> 3) + 8 * h + (r & 7);
}

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// The element e of an 8-pair block alone (both halves), as a mask on the packed block.
__device__ inline u32x4 pair_mask(int e) {
    u32x4 q;
#pragma unroll
    for (int t = 0; t < 4; ++t)
        q[t] = (e >> 1) == t ? ((e & 1) ? 0xffff0000u : 0xffffu) : 0u;
    return q;
}

// Leading nz pairs of an 8-pair block zeroed, as a mask on the packed block.
__device__ inline u32x4 lead_mask(int nz) {
    u32x4 q;
#pragma unroll
    for (int t = 0; t < 4; ++t)
        q[t] = ((2 * t >= nz) ? 0xffffu : 0u) | ((2 * t + 1 >= nz) ? 0xffff0000u : 0u);
    return q;
}

__device__ inline u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ inline f32x16 mfma_h(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ inline f32x16 mfma_b(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Registers 8s..8s+7 of a C block as a packed 16-deep operand (f16 or bf16).
template <bool BF>
__device__ inline u32x4 pack8(const f32x16& c, int s) {
    u32x4 o;
#pragma unroll
    for (int t = 0; t < 4; ++t)
        o[t] = BF ? pack_bf16x2(c[8 * s + 2 * t], c[8 * s + 2 * t + 1])
                  : pack_f16x2(c[8 * s + 2 * t], c[8 * s + 2 * t + 1]);
    return o;
}

// Pair of the row x (pair-block element order, x = 16j + e) of a 32-row block db.
__device__ inline int pair_of_x(int db, int x) { return 8 * (2 * db + (x >> 4)) + (x & 7); }

// Work index i of n (ordered by growing length) as the wave's two ranges: i and n-1-i take
// turns, so every wave holds one short and one long range.
__device__ inline int paired(int i, int n, int half) { return half ? n - 1 - i : i; }

// ---------------------------------------------------------------------------- prep kernels

template <int D>
__global__ __launch_bounds__(256) void bwd_prep_k_kernel(BwdParams p, Tables tab) {
    constexpr int P = D / 2, NB = D / 16;
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)p.B * p.Hkv * p.Np;
    if (id >= total) return;
    const int64_t t = id % p.Np;
    const int64_t bg = id / p.Np;
    uint16_t* ks = p.ks + bg * NB * p.Np * 16;
    uint16_t* vb = p.vb + bg * NB * p.Np * 16;
    // K'^T by key octets: element (x, t) at ((t/8) D + x) 8 + t%8
    uint16_t* kt = p.kt + bg * D * p.Np + (t >> 3) * D * 8 + (t & 7);
    if (t >= p.N) {
        for (int j = 0; j < NB; ++j) {
            u32x4* d4 = reinterpret_cast<u32x4*>(ks + ((int64_t)j * p.Np + t) * 16);
            d4[0] = u32x4{0u, 0u, 0u, 0u};
            d4[1] = u32x4{0u, 0u, 0u, 0u};
            u32x4* v4 = reinterpret_cast<u32x4*>(vb + ((int64_t)j * p.Np + t) * 16);
            v4[0] = u32x4{0u, 0u, 0u, 0u};
            v4[1] = u32x4{0u, 0u, 0u, 0u};
        }
        for (int x = 0; x < D; ++x) kt[x * 8] = 0;
        return;
    }
    const int g = (int)(bg % p.Hkv), b = (int)(bg / p.Hkv);
    const uint16_t* kr = static_cast<const uint16_t*>(p.k) + (((int64_t)b * p.N + t) * p.Hkv + g) * D;
    const uint16_t* vr = static_cast<const uint16_t*>(p.v) + (((int64_t)b * p.N + t) * p.Hkv + g) * D;
    for (int j = 0; j < NB; ++j) {
        const u32x4* s4 = reinterpret_cast<const u32x4*>(vr + 16 * j);
        u32x4* v4 = reinterpret_cast<u32x4*>(vb + ((int64_t)j * p.Np + t) * 16);
        v4[0] = s4[0];
        v4[1] = s4[1];
    }
    for (int j = 0; j < NB; ++j) {
        uint16_t el[16];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = 8 * j + e;
            const int ix = p.interleaved ? 2 * i : i, iy = p.interleaved ? 2 * i + 1 : i + P;
            const float x = bf16_bits_to_f32(kr[ix]), y = bf16_bits_to_f32(kr[iy]);
            float sn, cs;
            rope_sincos(t, tab.theta[i], &sn, &cs);
            el[e] = f32_to_f16_bits(x * cs - y * sn);
            el[8 + e] = f32_to_f16_bits(y * cs + x * sn);
        }
        u32x4 w0, w1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            w0[q] = (uint32_t)el[2 * q] | ((uint32_t)el[2 * q + 1] << 16);
            w1[q] = (uint32_t)el[8 + 2 * q] | ((uint32_t)el[8 + 2 * q + 1] << 16);
        }
        u32x4* d4 = reinterpret_cast<u32x4*>(ks + ((int64_t)j * p.Np + t) * 16);
        d4[0] = w0;
        d4[1] = w1;
#pragma unroll
        for (int e = 0; e < 16; ++e) kt[(16 * j + e) * 8] = el[e];
    }
}

template <int D>
__global__ __launch_bounds__(256) void bwd_prep_q_kernel(BwdParams p, Tables tab) {
    constexpr int P = D / 2, NB = D / 16;
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)p.B * p.Hq * p.Np;
    if (id >= total) return;
    const int64_t t = id % p.Np;
    const int64_t bh = id / p.Np;
    uint16_t* qs = p.qs + bh * NB * p.Np * 16;
    uint16_t* dob = p.dob + bh * NB * p.Np * 16;
    // Q'^T and dout^T by row octets: element (x, t) at ((t/8) D + x) 8 + t%8
    uint16_t* qt = p.qt + bh * D * p.Np + (t >> 3) * D * 8 + (t & 7);
    uint16_t* dot = p.dot + bh * D * p.Np + (t >> 3) * D * 8 + (t & 7);
    if (t >= p.N) {
        for (int j = 0; j < NB; ++j) {
            u32x4* d4 = reinterpret_cast<u32x4*>(qs + ((int64_t)j * p.Np + t) * 16);
            d4[0] = u32x4{0u, 0u, 0u, 0u};
            d4[1] = u32x4{0u, 0u, 0u, 0u};
            u32x4* g4 = reinterpret_cast<u32x4*>(dob + ((int64_t)j * p.Np + t) * 16);
            g4[0] = u32x4{0u, 0u, 0u, 0u};
            g4[1] = u32x4{0u, 0u, 0u, 0u};
        }
        for (int x = 0; x < D; ++x) {
            qt[x * 8] = 0;
            dot[x * 8] = 0;
        }
        p.lse2[bh * p.Np + t] = INFINITY;      // rows past the end: P = 0
        p.Dr[bh * p.Np + t] = 0.f;
        return;
    }
    const int h = (int)(bh % p.Hq), b = (int)(bh / p.Hq);
    const int64_t row = (((int64_t)b * p.N + t) * p.Hq + h) * D;
    const uint16_t* qr = static_cast<const uint16_t*>(p.q) + row;
    const float sl2 = p.scale * kLog2e;
    for (int j = 0; j < NB; ++j) {
        uint16_t es[16], eu[16];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = 8 * j + e;
            const int ix = p.interleaved ? 2 * i : i, iy = p.interleaved ? 2 * i + 1 : i + P;
            const float x = bf16_bits_to_f32(qr[ix]), y = bf16_bits_to_f32(qr[iy]);
            float sn, cs;
            rope_sincos(t, tab.theta[i], &sn, &cs);
            const float rx = x * cs - y * sn, ry = y * cs + x * sn;
            es[e] = f32_to_f16_bits(rx * sl2);
            es[8 + e] = f32_to_f16_bits(ry * sl2);
            eu[e] = f32_to_f16_bits(rx);
            eu[8 + e] = f32_to_f16_bits(ry);
        }
        u32x4 w0, w1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            w0[q] = (uint32_t)es[2 * q] | ((uint32_t)es[2 * q + 1] << 16);
            w1[q] = (uint32_t)es[8 + 2 * q] | ((uint32_t)es[8 + 2 * q + 1] << 16);
        }
        u32x4* d4 = reinterpret_cast<u32x4*>(qs + ((int64_t)j * p.Np + t) * 16);
        d4[0] = w0;
        d4[1] = w1;
#pragma unroll
        for (int e = 0; e < 16; ++e) qt[(16 * j + e) * 8] = eu[e];
    }
    // dout blocked and by row octets (natural dim order), and D = dout . out
    const uint16_t* gr = static_cast<const uint16_t*>(p.dout) + row;
    for (int j = 0; j < NB; ++j) {
        const u32x4* s4 = reinterpret_cast<const u32x4*>(gr + 16 * j);
        u32x4* g4 = reinterpret_cast<u32x4*>(dob + ((int64_t)j * p.Np + t) * 16);
        g4[0] = s4[0];
        g4[1] = s4[1];
    }
    float dd = 0.f;
    for (int x = 0; x < D; ++x) {
        const uint16_t gb = gr[x];
        dot[x * 8] = gb;
        const float o = p.out_f32 ? static_cast<const float*>(p.out)[row + x]
                                  : bf16_bits_to_f32(static_cast<const uint16_t*>(p.out)[row + x]);
        dd += bf16_bits_to_f32(gb) * o;
    }
    p.Dr[bh * p.Np + t] = dd;
    p.lse2[bh * p.Np + t] = p.lse[((int64_t)b * p.Hq + h) * p.N + t] * kLog2e;
}

// ---------------------------------------------------------------------------- dq

// dq: a workgroup takes Gc q heads x R row groups (32 rows each) of one kv head and streams
// that kv head's key tiles through LDS: K' (pair-blocked), V (blocked by 16 dims) and K'^T
// (by key octets), each one contiguous copy per tile, loaded by an extra producer wave into a
// two-stage ring.  Every K/V byte then leaves memory once per workgroup.
template <int D>
struct DqTile {
    static constexpr int BN = D == 64 ? 128 : 64;       // keys per tile (3 BN d 2 bytes a stage)
    static constexpr int NSUB = BN / 32;
    static constexpr int MAXW = 7;                      // compute waves per workgroup
};

template <int D>
__global__ __launch_bounds__(64 * (DqTile<D>::MAXW + 1)) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_kernel(BwdParams p, Tables tab, BwdLaunch L) {
    constexpr int NB = D / 16, NDB = D / 32, P = D / 2, BN = DqTile<D>::BN, NSUB = DqTile<D>::NSUB;
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][NB * BN * 16];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][NB * BN * 16];
    __shared__ __attribute__((aligned(16))) uint16_t sT[2][BN * D];
    const int tid = threadIdx.x;
    const int w = uniform(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, h = lane >> 5;
    const int G = p.Hq / p.Hkv;
    const int U = p.B * p.Hkv * L.nhc;
    const int u = blockIdx.x % U;
    const int rb = L.n_rb - 1 - (int)(blockIdx.x / U);     // longest rows first
    const int hc = u % L.nhc, g = (u / L.nhc) % p.Hkv, b = u / (L.nhc * p.Hkv);
    const int hin = hc * L.Gc + (w % L.Gc), rg = w / L.Gc;
    const bool producer = w == L.Gc * L.R;
    const int qs0 = rb * 32 * L.R;
    const int q0 = qs0 + 32 * rg;
    const bool wave_ok = !producer && hin < G && q0 < p.N;
    const int hq = g * G + (hin < G ? hin : 0);
    const int bh = b * p.Hq + hq;
    const int row_end = (qs0 + 32 * L.R < p.N ? qs0 + 32 * L.R : (int)p.N) - 1;
    const int kt_last = row_end / BN;
    const int64_t kvh = (int64_t)b * p.Hkv + g;
    const uint16_t* ksg = p.ks + kvh * NB * p.Np * 16;
    const uint16_t* vbg = p.vb + kvh * NB * p.Np * 16;
    const uint16_t* ktg = p.kt + kvh * D * p.Np;
    const float sc = p.scale;

    // tile kt into stage st: K' and V block j are BN rows of 32 bytes (BN/32 wave loads of
    // 1 KB each); the K'^T octets of the tile are BN*D*2 contiguous bytes.  Pair blocks below
    // jlo, dead for every row of the workgroup at the tile's smallest distance, are not
    // loaded: no wave reads K' there, and their K'^T dims enter the dq product only as the
    // zeroed operand of inactive dims.  (A K'^T wave load holds 64 dims of one octet.)
    // (the producer's band edge lives in LDS: a register would be held by every wave)
    __shared__ int s_plo;
    auto issue = [&](int kt, int st) {
        const int64_t k0 = (int64_t)kt * BN;
        const int dmin = uniform(qs0 - (int)(k0 + BN - 1) > 0 ? qs0 - (int)(k0 + BN - 1) : 0);
        int plo_wg = kt == kt_last ? 0 : uniform(s_plo);
        while (plo_wg < P && tab.W[plo_wg] < dmin) ++plo_wg;
        s_plo = plo_wg;
        const int jlo = plo_wg >> 3;
        for (int j = 0; j < NB; ++j)
            for (int part = 0; part < BN / 32; ++part) {
                const int64_t off = ((int64_t)j * p.Np + k0 + 32 * part) * 16 + lane * 8;
                if (j >= jlo)
                    __builtin_amdgcn_global_load_lds(ksg + off, (lds_ptr)&sK[st][(j * BN + 32 * part) * 16], 16, 0, 0);
                __builtin_amdgcn_global_load_lds(vbg + off, (lds_ptr)&sV[st][(j * BN + 32 * part) * 16], 16, 0, 0);
            }
        for (int i = 0; i < BN * D * 2 / 1024; ++i)
            if (64 * (i % (D / 64)) + 63 >= 16 * jlo)
                __builtin_amdgcn_global_load_lds(ktg + k0 * D + (i * 64 + lane) * 8, (lds_ptr)&sT[st][i * 512],
                                                 16, 0, 0);
    };

    // this wave's rows (lane = row): Q' (scaled) and dout as B operands, lse2 and D
    const int row = q0 + l32;
    const bool row_ok = wave_ok && row < p.N;
    const int rowc = row < p.N ? row : (int)p.N - 1;
    u32x4 Qb[NB], Gb[NB];
    float lse2 = 0.f, Dv = 0.f;
    f32x16 acc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};
    if (wave_ok) {
        const uint16_t* qsh = p.qs + (int64_t)bh * NB * p.Np * 16;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            Qb[j] = ld16(qsh + ((int64_t)j * p.Np + row) * 16 + 8 * h);
            Gb[j] = ld16(static_cast<const uint16_t*>(p.dout) +
                         (((int64_t)b * p.N + rowc) * p.Hq + hq) * D + 16 * j + 8 * h);
        }
        lse2 = p.lse2[(int64_t)bh * p.Np + row];
        Dv = p.Dr[(int64_t)bh * p.Np + row];
    }
    int plo = 0, pfull = 0;                             // band edges, distances only grow

    auto compute = [&](int kt, const uint16_t* cK, const uint16_t* cV, const uint16_t* cT) {
        for (int sub = NSUB - 1; sub >= 0; --sub) {
            const int c0 = kt * BN + 32 * sub;
            if (c0 > q0 + 31) continue;                 // above every row of the wave
            const int dmin = uniform(q0 - (c0 + 31) > 0 ? q0 - (c0 + 31) : 0);
            const int dmax = uniform(q0 + 31 - c0);
            while (plo < P && tab.W[plo] < dmin) ++plo;
            while (pfull < P && tab.W[pfull] < dmax) ++pfull;
            if (pfull < plo) pfull = plo;
            const int krow = 32 * sub + perm_row(l32);  // key (in the tile) this lane feeds to A
            auto K = [&](int j) { return ld16(cK + (j * BN + krow) * 16 + 8 * h); };
            auto V = [&](int j) { return ld16(cV + (j * BN + krow) * 16 + 8 * h); };
            // K'^T rows x, keys 16s + 8h .. +7 of the sub-tile: octet 4 sub + 2 s + h
            auto T = [&](int db, int s2) { return ld16(cT + ((4 * sub + 2 * s2 + h) * D + 32 * db + l32) * 8); };
            // dP^T = V dout^T first: it does not wait on the scores, so its operand reads and
            // MFMAs overlap the score chain's
            f32x16 dPt = f32x16{};
#pragma unroll
            for (int j = 0; j < NB; ++j) dPt = mfma_b(V(j), Gb[j], dPt);
            // S^T (log2 units): straddling pairs one by one, then the fully active blocks;
            // register r of half h holds key c0 + idx(r); distance = row - key
            f32x16 S = f32x16{};
            for (int e = plo; e < pfull; ++e) {
                S = mfma_h(K(e >> 3), Qb[e >> 3] & pair_mask(e & 7), S);
                const int We = tab.W[e];
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (row - (c0 + idx_of_reg(r, h)) > We) S[r] = 0.f;
            }
            const int jf = pfull >> 3;
            // unrolled over the blocks with a uniform test each: a block index known at compile
            // time keeps Qb in place (a run-time index into it became indexed register moves)
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                if (j < jf) continue;
                const u32x4 qb = j == jf ? (Qb[j] & lead_mask(pfull - 8 * jf)) : Qb[j];
                S = mfma_h(K(j), qb, S);
            }
            // the dq product's K'^T operands of the upper dim blocks (the ones long distances
            // keep), read before the exponentials so that their latency passes under them
            u32x4 Tpre[NDB / 2][2];
#pragma unroll
            for (int i = 0; i < NDB / 2; ++i)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) Tpre[i][s2] = T(NDB / 2 + i, s2);
            // P^T, dP^T, dl^T (lane = row; register = key).  Only a sub-tile that crosses the
            // diagonal needs the causal test; rows past the end hold lse2 = +inf (P = 0).
            f32x16 Pt;
            if (c0 + 31 > q0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = c0 + idx_of_reg(r, h);
                    Pt[r] = key <= row ? __builtin_amdgcn_exp2f(S[r] - lse2) : 0.f;
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) Pt[r] = __builtin_amdgcn_exp2f(S[r] - lse2);
            }
            f32x16 dl;
#pragma unroll
            for (int r = 0; r < 16; ++r) dl[r] = Pt[r] * (dPt[r] - Dv);
            // dq'^T += K'^T dl^T over the fully active pairs' dims (block db holds pairs 16db ..
            // 16db + 15: only the block holding the band edge has inactive dims to zero) ...
            const u32x4 dlb[2] = {pack8<false>(dl, 0), pack8<false>(dl, 1)};
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                if (16 * db + 15 < pfull) continue;     // every dim of this block dead or straddling
                auto Top = [&](int s2) { return db >= NDB / 2 ? Tpre[db - NDB / 2][s2] : T(db, s2); };
                if (16 * db >= pfull) {
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) acc[db] = mfma_h(Top(s2), dlb[s2], acc[db]);
                } else {
                    const bool on = pair_of_x(db, l32) >= pfull;
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        u32x4 a = Top(s2);
                        if (!on) a = u32x4{0u, 0u, 0u, 0u};
                        acc[db] = mfma_h(a, dlb[s2], acc[db]);
                    }
                }
            }
            // ... and each straddling pair with dl masked to its window
            for (int e = plo; e < pfull; ++e) {
                const int We = tab.W[e];
                f32x16 m;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    m[r] = (row - (c0 + idx_of_reg(r, h)) <= We) ? dl[r] : 0.f;
                const int db = e >> 4;
                const bool on = pair_of_x(db, l32) == e;
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    u32x4 a = T(db, s2);
                    if (!on) a = u32x4{0u, 0u, 0u, 0u};
                    // (db is wave-uniform: select the accumulator without indexing)
#pragma unroll
                    for (int dd = 0; dd < NDB; ++dd)
                        if (dd == db) acc[dd] = mfma_h(a, pack8<false>(m, s2), acc[dd]);
                }
            }
        }
    };

    // The producer streams tile kt-1 into one stage while the others compute tile kt from
    // the other; it waits for its own loads before the barrier that hands the stage over.
    if (producer) {
        issue(kt_last, 0);
        __builtin_amdgcn_s_waitcnt(0x0070);             // vmcnt(0) lgkmcnt(0)
    }
    for (int kt = kt_last, it = 0; kt >= 0; --kt, ++it) {
        __syncthreads();
        if (producer) {
            if (kt > 0) {
                issue(kt - 1, (it & 1) ^ 1);
                __builtin_amdgcn_s_waitcnt(0x0070);
            }
        } else if (wave_ok) {
            compute(kt, sK[it & 1], sV[it & 1], sT[it & 1]);
        }
    }

    // epilogue: scale, rotate back at the row's position, write dq (lane = row)
    if (row_ok) {
        const int64_t ob = (((int64_t)b * p.N + row) * p.Hq + hq) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if ((r >> 2) & 1) continue;             // y-components: with their x
                const int xl = 8 * (r >> 2) + 4 * h + (r & 3);
                const int i = 8 * (2 * db + (xl >> 4)) + (xl & 7);
                float sn, cs;
                rope_sincos(row, tab.theta[i], &sn, &cs);
                const float gx = acc[db][r] * sc, gy = acc[db][r + 4] * sc;
                const float ox = gx * cs + gy * sn, oy = gy * cs - gx * sn;
                const int ix = p.interleaved ? 2 * i : i, iy = p.interleaved ? 2 * i + 1 : i + P;
                if (p.grad_f32) {
                    static_cast<float*>(p.dq)[ob + ix] = ox;
                    static_cast<float*>(p.dq)[ob + iy] = oy;
                } else {
                    static_cast<uint16_t*>(p.dq)[ob + ix] = f32_to_bf16_bits(ox);
                    static_cast<uint16_t*>(p.dq)[ob + iy] = f32_to_bf16_bits(oy);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------- dk, dv

// dk, dv: a workgroup takes R key groups (32 keys each) of one q head and streams that q
// head's row tiles through LDS: Q' (pair-blocked, scaled), dout (blocked by 16 dims), Q'^T
// and dout^T (by row octets), and the rows' lse and D; the producer wave fills a two-stage
// ring.  Each compute wave keeps its keys' K' and V as B operands and its dk'^T, dv^T
// accumulators in registers, and writes them per q head to the workspace.  (At d = 128 one
// kernel with both accumulators fit 5 compute waves per CU; the two passes, 11 and 7 waves,
// took 292 ms against 328 for the Llama-3.2-3B shape at 128K though both compute the scores.)
template <int D, int PASS>
struct DkTile {
    // PASS 0: dk and dv in one kernel (d = 64).  d = 128 takes two passes, 1: dv only, 2: dk
    // only; each carries half the accumulators and half the row tiles' arrays, so more waves
    // fit in a CU's registers and LDS than the 5 of one combined kernel.
    static constexpr int BM = D == 64 ? 128 : 64;       // rows per tile
    static constexpr int NSUB = BM / 32;
    static constexpr int MAXW = D == 64 ? 7 : (PASS == 1 ? 11 : 7);   // compute waves per workgroup
    static constexpr int WPE = PASS == 1 ? 3 : 2;                      // waves per SIMD to fit
};

template <int D, int PASS>
__global__ __launch_bounds__(64 * (DkTile<D, PASS>::MAXW + 1))
__attribute__((amdgpu_waves_per_eu(DkTile<D, PASS>::WPE)))
void bwd_dkdv_kernel(BwdParams p, Tables tab, int R) {
    constexpr int NB = D / 16, NDB = D / 32, P = D / 2, BM = DkTile<D, PASS>::BM;
    constexpr int NSUB = DkTile<D, PASS>::NSUB, MAXW = DkTile<D, PASS>::MAXW;
    constexpr bool DO_DV = PASS != 2, DO_DK = PASS != 1;
    // the row tiles' arrays a pass reads (one that does not read an array declares a stub)
    __shared__ __attribute__((aligned(16))) uint16_t sQ[2][NB * BM * 16];
    __shared__ __attribute__((aligned(16))) uint16_t sG[2][DO_DK ? NB * BM * 16 : 8];
    __shared__ __attribute__((aligned(16))) uint16_t sQt[2][DO_DK ? BM * D : 8];
    __shared__ __attribute__((aligned(16))) uint16_t sGt[2][DO_DV ? BM * D : 8];
    __shared__ __attribute__((aligned(16))) float sL[2][2 * BM];     // lse2, then D, of the rows
    // d = 128: each compute wave's keys' K' (pair-blocked, 32 rows of 32 bytes per block), the B
    // operand of S, copied once into LDS (held in registers it spills; read from L2 per
    // sub-tile its latency stalls the S chain).  V, the B operand of dP, sits in LDS too when
    // one kernel does both products, in registers in the dk pass, and is not read by the dv pass.
    constexpr bool KLDS = D == 128;
    constexpr bool VLDS = D == 128 && PASS == 0, VHOLD = D == 128 && PASS == 2;
    __shared__ __attribute__((aligned(16))) uint16_t sKw[KLDS ? MAXW : 1][KLDS ? NB * 32 * 16 : 8];
    __shared__ __attribute__((aligned(16))) uint16_t sVw[VLDS ? MAXW : 1][VLDS ? NB * 32 * 16 : 8];
    const int tid = threadIdx.x;
    const int w = uniform(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, h = lane >> 5;
    const int U = p.B * p.Hq;
    const int bh = blockIdx.x % U;
    const int kbk = (int)(blockIdx.x / U);              // key blocks with the most rows first
    const int hq = bh % p.Hq, b = bh / p.Hq;
    const int g = hq / (p.Hq / p.Hkv);
    const bool producer = w == R;
    const int c0 = 32 * (kbk * R + w);                  // this wave's first key
    const bool wave_ok = !producer && c0 < p.N;
    const int key = c0 + l32;
    const int keyc = key < p.N ? key : (int)p.N - 1;
    const int nrt = (int)((p.N + BM - 1) / BM);
    const int rt_first = (32 * kbk * R) / BM;           // the tile holding the first key's row
    const uint16_t* qsh = p.qs + (int64_t)bh * NB * p.Np * 16;
    const uint16_t* gbh = p.dob + (int64_t)bh * NB * p.Np * 16;
    const uint16_t* qth = p.qt + (int64_t)bh * D * p.Np;
    const uint16_t* gth = p.dot + (int64_t)bh * D * p.Np;
    const float* lse2h = p.lse2 + (int64_t)bh * p.Np;
    const float* Drh = p.Dr + (int64_t)bh * p.Np;

    // row tile rt into stage st: Q' and dout block j are BM rows of 32 bytes (BM/32 wave loads
    // of 1 KB), the octet arrays BM*D*2 contiguous bytes, lse2 and D BM floats each
    // (pair blocks below jlo, dead for every key of the workgroup at the tile's smallest
    // distance: Q' and the Q'^T dims of whole dead wave loads are not loaded, as in dq)
    // (the producer's band edge lives in LDS: a register would be held by every wave)
    __shared__ int s_plo;
    auto issue = [&](int rt, int st) {
        const int64_t r0 = (int64_t)rt * BM;
        const int kend_wg = 32 * (kbk * R + R) - 1;     // the workgroup's last key
        const int dmin = uniform((int)r0 - kend_wg > 0 ? (int)r0 - kend_wg : 0);
        int plo_wg = rt == rt_first ? 0 : uniform(s_plo);
        while (plo_wg < P && tab.W[plo_wg] < dmin) ++plo_wg;
        s_plo = plo_wg;
        const int jlo = plo_wg >> 3;
        for (int j = 0; j < NB; ++j)
            for (int part = 0; part < BM / 32; ++part) {
                const int64_t off = ((int64_t)j * p.Np + r0 + 32 * part) * 16 + lane * 8;
                if (j >= jlo)
                    __builtin_amdgcn_global_load_lds(qsh + off, (lds_ptr)&sQ[st][(j * BM + 32 * part) * 16], 16, 0, 0);
                if constexpr (DO_DK)
                    __builtin_amdgcn_global_load_lds(gbh + off, (lds_ptr)&sG[st][(j * BM + 32 * part) * 16], 16, 0, 0);
            }
        for (int i = 0; i < BM * D * 2 / 1024; ++i) {
            const int64_t off = r0 * D + (i * 64 + lane) * 8;
            if constexpr (DO_DK)
                __builtin_amdgcn_global_load_lds(qth + off, (lds_ptr)&sQt[st][i * 512], 16, 0, 0);
            if constexpr (DO_DV)
                __builtin_amdgcn_global_load_lds(gth + off, (lds_ptr)&sGt[st][i * 512], 16, 0, 0);
        }
        if constexpr (BM >= 64) {
            for (int i = 0; i < BM / 64; ++i) {
                __builtin_amdgcn_global_load_lds(lse2h + r0 + 64 * i + lane, (lds_ptr)&sL[st][64 * i], 4, 0, 0);
                __builtin_amdgcn_global_load_lds(Drh + r0 + 64 * i + lane, (lds_ptr)&sL[st][BM + 64 * i], 4, 0, 0);
            }
        } else {
            // 32 rows: lanes 0-31 bring lse2, lanes 32-63 D, in one load
            static_assert(BM == 32, "row statistics of a 32-row tile fill one wave load");
            const float* src = lane < 32 ? lse2h + r0 + lane : Drh + r0 + (lane - 32);
            __builtin_amdgcn_global_load_lds(src, (lds_ptr)&sL[st][0], 4, 0, 0);
        }
    };

    // this wave's keys (lane = key): K' and V, the B operands of S and dP.  V is read again from
    // the workspace (L2) each sub-tile, its loads issued ahead of the products; so is K' at
    // d = 128, where holding it next to the dk'^T, dv^T accumulators spills (measured: 923 ms
    // against 1001 ms for the Llama-3.2-3B shape at 128K); at d = 64 it is held (14.3 against
    // 13.3 ms for the Qwen2.5-0.5B shape at 32K).
    constexpr bool HOLDK = D == 64;
    u32x4 Kh[HOLDK ? NB : 1];
    u32x4 Vh[VHOLD ? NB : 1];
    static_assert(HOLDK != KLDS, "K' is held in registers at d = 64 and in LDS at d = 128");
    f32x16 dK[NDB], dV[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
        dK[i] = f32x16{};
        dV[i] = f32x16{};
    }
    const int64_t kvh = (int64_t)b * p.Hkv + g;
    const uint16_t* kkey = p.ks + (kvh * NB * p.Np + key) * 16 + 8 * h;
    const uint16_t* vkey = p.vb + (kvh * NB * p.Np + key) * 16 + 8 * h;
    if constexpr (HOLDK) {
        if (wave_ok) {
#pragma unroll
            for (int j = 0; j < NB; ++j) Kh[j] = ld16(kkey + (int64_t)j * p.Np * 16);
        }
    }
    if constexpr (VHOLD) {
        if (wave_ok) {
#pragma unroll
            for (int j = 0; j < NB; ++j) Vh[j] = ld16(vkey + (int64_t)j * p.Np * 16);
        }
    }
    if constexpr (KLDS) {
        // block j's 32 rows are 1 KB of the workspace: one direct load per block, landed before
        // the tile loop (so no compute wave has a direct load in flight inside it)
        if (wave_ok) {
            const uint16_t* k0 = p.ks + (kvh * NB * p.Np + c0) * 16;
            const uint16_t* v0 = p.vb + (kvh * NB * p.Np + c0) * 16;
            for (int j = 0; j < NB; ++j) {
                __builtin_amdgcn_global_load_lds(k0 + (int64_t)j * p.Np * 16 + lane * 8,
                                                 (lds_ptr)&sKw[w][j * 512], 16, 0, 0);
                if constexpr (VLDS)
                    __builtin_amdgcn_global_load_lds(v0 + (int64_t)j * p.Np * 16 + lane * 8,
                                                     (lds_ptr)&sVw[w][j * 512], 16, 0, 0);
            }
            __builtin_amdgcn_s_waitcnt(0x0070);
        }
    }
    int plo = 0, pfull = 0;                             // band edges, distances only grow

    auto compute = [&](int rt, const uint16_t* cQ, const uint16_t* cG, const uint16_t* cQt,
                       const uint16_t* cGt, const float* cL) {
        for (int sub = 0; sub < NSUB; ++sub) {
            const int r0 = rt * BM + 32 * sub;
            if (r0 + 31 < c0 || r0 >= p.N) continue;    // rows before every key, or past the end
            const int dmin = uniform(r0 - (c0 + 31) > 0 ? r0 - (c0 + 31) : 0);
            const int dmax = uniform(r0 + 31 - c0);
            while (plo < P && tab.W[plo] < dmin) ++plo;
            while (pfull < P && tab.W[pfull] < dmax) ++pfull;
            if (pfull < plo) pfull = plo;
            const int arow = 32 * sub + perm_row(l32);  // row (in the tile) this lane feeds to A
            u32x4 Kb[NB], Vb[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                if constexpr (HOLDK) {
                    Kb[j] = Kh[j];
                    Vb[j] = ld16(vkey + (int64_t)j * p.Np * 16);
                } else {
                    Kb[j] = ld16(&sKw[w][(j * 32 + l32) * 16 + 8 * h]);
                    if constexpr (VLDS) Vb[j] = ld16(&sVw[w][(j * 32 + l32) * 16 + 8 * h]);
                    else if constexpr (VHOLD) Vb[j] = Vh[j];
                    else Vb[j] = u32x4{0u, 0u, 0u, 0u};       // the dv pass has no dP
                }
            }
            auto Q = [&](int j) { return ld16(cQ + (j * BM + arow) * 16 + 8 * h); };
            auto Gr = [&](int j) { return ld16(cG + (j * BM + arow) * 16 + 8 * h); };
            // x^T rows x, rows 16s + 8h .. +7 of the sub-tile: octet 4 sub + 2 s + h
            auto QT = [&](int db, int s2) { return ld16(cQt + ((4 * sub + 2 * s2 + h) * D + 32 * db + l32) * 8); };
            auto GT = [&](int db, int s2) { return ld16(cGt + ((4 * sub + 2 * s2 + h) * D + 32 * db + l32) * 8); };
            // dP = dout V^T (A = dout rows, permuted), first: it does not wait on the scores
            f32x16 dP = f32x16{};
            if constexpr (DO_DK) {
#pragma unroll
                for (int j = 0; j < NB; ++j) dP = mfma_b(Gr(j), Vb[j], dP);
            }
            // S (log2 units): register r of half h holds row r0 + idx(r); distance = row - key
            f32x16 S = f32x16{};
            for (int e = plo; e < pfull; ++e) {
                S = mfma_h(Q(e >> 3), Kb[e >> 3] & pair_mask(e & 7), S);
                const int We = tab.W[e];
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if ((r0 + idx_of_reg(r, h)) - key > We) S[r] = 0.f;
            }
            const int jf = pfull >> 3;
            // unrolled over the blocks with a uniform test each (Kb indexed at compile time)
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                if (j < jf) continue;
                const u32x4 kb = j == jf ? (Kb[j] & lead_mask(pfull - 8 * jf)) : Kb[j];
                S = mfma_h(Q(j), kb, S);
            }
            // lse and D of this lane's 16 rows: 32 sub + 8h + 0..7 and 32 sub + 16 + 8h + 0..7
            const f32x4* l4 = reinterpret_cast<const f32x4*>(cL + 32 * sub + 8 * h);
            const f32x4* d4 = reinterpret_cast<const f32x4*>(cL + BM + 32 * sub + 8 * h);
            const f32x4 la = l4[0], lb = l4[1], lc = l4[4], ld = l4[5];
            const f32x4 da = d4[0], dbv = d4[1], dc = d4[4], dd = d4[5];
            auto lse_r = [&](int r) { const f32x4& v = r < 4 ? la : (r < 8 ? lb : (r < 12 ? lc : ld)); return v[r & 3]; };
            auto D_r = [&](int r) { const f32x4& v = r < 4 ? da : (r < 8 ? dbv : (r < 12 ? dc : dd)); return v[r & 3]; };
            // only a sub-tile that crosses the diagonal needs the causal test; rows past the
            // end hold lse2 = +inf (P = 0)
            f32x16 Pm;
            if (r0 < c0 + 31) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = r0 + idx_of_reg(r, h);
                    Pm[r] = key <= row ? __builtin_amdgcn_exp2f(S[r] - lse_r(r)) : 0.f;
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) Pm[r] = __builtin_amdgcn_exp2f(S[r] - lse_r(r));
            }
            f32x16 dl = f32x16{};
            if constexpr (DO_DK) {
#pragma unroll
                for (int r = 0; r < 16; ++r) dl[r] = Pm[r] * (dP[r] - D_r(r));
            }
            // dv^T += dout^T P ; dk'^T += Q'^T dl (fully active pairs' dims, then straddling).
            // P enters the dv product as two bf16 parts, P = hi + lo: a key's dv sums the
            // probabilities of every row of every q head of its kv head (an early key's reaches
            // ~10 and more), where one bf16 rounding of P alone would cost ~2e-2 max-abs.
            if constexpr (DO_DV) {
                f32x16 Plo;
#pragma unroll
                for (int r = 0; r < 16; ++r) Plo[r] = Pm[r] - round_bf16(Pm[r]);
                const u32x4 pb[2] = {pack8<true>(Pm, 0), pack8<true>(Pm, 1)};
                const u32x4 pl[2] = {pack8<true>(Plo, 0), pack8<true>(Plo, 1)};
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        const u32x4 a = GT(db, s2);
                        dV[db] = mfma_b(a, pb[s2], dV[db]);
                        dV[db] = mfma_b(a, pl[s2], dV[db]);
                    }
                }
            }
            if constexpr (DO_DK) {
                const u32x4 dlb[2] = {pack8<false>(dl, 0), pack8<false>(dl, 1)};
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    if (16 * db + 15 < pfull) continue;     // every dim dead or straddling
                    if (16 * db >= pfull) {                 // every dim active
#pragma unroll
                        for (int s2 = 0; s2 < 2; ++s2) dK[db] = mfma_h(QT(db, s2), dlb[s2], dK[db]);
                    } else {
                        const bool on = pair_of_x(db, l32) >= pfull;
#pragma unroll
                        for (int s2 = 0; s2 < 2; ++s2) {
                            u32x4 a = QT(db, s2);
                            if (!on) a = u32x4{0u, 0u, 0u, 0u};
                            dK[db] = mfma_h(a, dlb[s2], dK[db]);
                        }
                    }
                }
                for (int e = plo; e < pfull; ++e) {
                    const int We = tab.W[e];
                    f32x16 m;
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        m[r] = ((r0 + idx_of_reg(r, h)) - key <= We) ? dl[r] : 0.f;
                    const int db = e >> 4;
                    const bool on = pair_of_x(db, l32) == e;
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        u32x4 a = QT(db, s2);
                        if (!on) a = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                        for (int dd2 = 0; dd2 < NDB; ++dd2)
                            if (dd2 == db) dK[dd2] = mfma_h(a, pack8<false>(m, s2), dK[dd2]);
                    }
                }
            }
        }
    };

    if (producer) {
        issue(rt_first, 0);
        __builtin_amdgcn_s_waitcnt(0x0070);             // vmcnt(0) lgkmcnt(0)
    }
    for (int rt = rt_first, it = 0; rt < nrt; ++rt, ++it) {
        __syncthreads();
        if (producer) {
            if (rt + 1 < nrt) {
                issue(rt + 1, (it & 1) ^ 1);
                __builtin_amdgcn_s_waitcnt(0x0070);
            }
        } else if (wave_ok) {
            compute(rt, sQ[it & 1], sG[it & 1], sQt[it & 1], sGt[it & 1], sL[it & 1]);
        }
    }
    if (!wave_ok) return;
    // this q head's dk'^T (unscaled, pair-block order) and dv^T for the lane's key, as fp32
    // partials [B][Hq][Np][d]; register r of half h holds x = 32db + 8(r/4) + 4h + r%4
    float* kp = p.dkp + ((int64_t)bh * p.Np + key) * D;
    float* vp = p.dvp + ((int64_t)bh * p.Np + key) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int x = 32 * db + 8 * q4 + 4 * h;
            if constexpr (DO_DK)
                *reinterpret_cast<f32x4*>(kp + x) = f32x4{dK[db][4 * q4], dK[db][4 * q4 + 1], dK[db][4 * q4 + 2], dK[db][4 * q4 + 3]};
            if constexpr (DO_DV)
                *reinterpret_cast<f32x4*>(vp + x) = f32x4{dV[db][4 * q4], dV[db][4 * q4 + 1], dV[db][4 * q4 + 2], dV[db][4 * q4 + 3]};
        }
    }
}

// dk, dv of every kv head: the sum over its q heads' partials; dk' scaled and rotated back.
template <int D>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdParams p, Tables tab) {
    constexpr int P = D / 2;
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)p.B * p.Hkv * p.N * P;
    if (id >= total) return;
    const int i = (int)(id % P);
    int64_t rest = id / P;
    const int64_t t = rest % p.N;
    rest /= p.N;
    const int g = (int)(rest % p.Hkv), b = (int)(rest / p.Hkv);
    const int G = p.Hq / p.Hkv;
    const int xk = 16 * (i >> 3) + (i & 7), yk = xk + 8;     // pair i in pair-block order
    const int ix = p.interleaved ? 2 * i : i, iy = p.interleaved ? 2 * i + 1 : i + P;
    float kx = 0.f, ky = 0.f, vx = 0.f, vy = 0.f;
    for (int hh = 0; hh < G; ++hh) {
        const int64_t base = (((int64_t)b * p.Hq + g * G + hh) * p.Np + t) * D;
        kx += p.dkp[base + xk];
        ky += p.dkp[base + yk];
        vx += p.dvp[base + ix];
        vy += p.dvp[base + iy];
    }
    float sn, cs;
    rope_sincos(t, tab.theta[i], &sn, &cs);
    kx *= p.scale;
    ky *= p.scale;
    const float ox = kx * cs + ky * sn, oy = ky * cs - kx * sn;
    const int64_t ob = (((int64_t)b * p.N + t) * p.Hkv + g) * D;
    if (p.grad_f32) {
        static_cast<float*>(p.dk)[ob + ix] = ox;
        static_cast<float*>(p.dk)[ob + iy] = oy;
        static_cast<float*>(p.dv)[ob + ix] = vx;
        static_cast<float*>(p.dv)[ob + iy] = vy;
    } else {
        static_cast<uint16_t*>(p.dk)[ob + ix] = f32_to_bf16_bits(ox);
        static_cast<uint16_t*>(p.dk)[ob + iy] = f32_to_bf16_bits(oy);
        static_cast<uint16_t*>(p.dv)[ob + ix] = f32_to_bf16_bits(vx);
        static_cast<uint16_t*>(p.dv)[ob + iy] = f32_to_bf16_bits(vy);
    }
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, const Tables& t, hipStream_t s) {
    const dim3 blk(256);
    const int64_t nk = (int64_t)p.B * p.Hkv * p.Np, nq = (int64_t)p.B * p.Hq * p.Np;
    bwd_prep_k_kernel<D><<<dim3((unsigned)((nk + 255) / 256)), blk, 0, s>>>(p, t);
    bwd_prep_q_kernel<D><<<dim3((unsigned)((nq + 255) / 256)), blk, 0, s>>>(p, t);
    const int64_t ngroups = (p.N + 31) / 32;
    // dq: Gc q heads x R row groups of one kv head per workgroup (plus the producer wave)
    const int G = p.Hq / p.Hkv, MW = DqTile<D>::MAXW;
    BwdLaunch L;
    L.nhc = (G + MW - 1) / MW;
    L.Gc = (G + L.nhc - 1) / L.nhc;
    L.R = MW / L.Gc > 1 ? MW / L.Gc : 1;
    L.n_rb = (int)((ngroups + L.R - 1) / L.R);
    const dim3 gq((unsigned)((int64_t)L.n_rb * p.B * p.Hkv * L.nhc)), bq(64 * (L.Gc * L.R + 1));
    bwd_dq_kernel<D><<<gq, bq, 0, s>>>(p, t, L);
    // dk, dv: R key groups of one q head per workgroup (plus the producer wave); at d = 128 a
    // dv pass, then a dk pass
    auto dkdv = [&](auto pass) {
        constexpr int PASS = decltype(pass)::value;
        const int RK = DkTile<D, PASS>::MAXW;
        const int64_t nkb = (ngroups + RK - 1) / RK;
        bwd_dkdv_kernel<D, PASS><<<dim3((unsigned)(nkb * p.B * p.Hq)), dim3(64 * (RK + 1)), 0, s>>>(p, t, RK);
    };
    if constexpr (D == 64) {
        dkdv(std::integral_constant<int, 0>{});
    } else {
        dkdv(std::integral_constant<int, 1>{});
        dkdv(std::integral_constant<int, 2>{});
    }
    const int64_t nr = (int64_t)p.B * p.Hkv * p.N * (D / 2);
    bwd_reduce_kernel<D><<<dim3((unsigned)((nr + 255) / 256)), blk, 0, s>>>(p, t);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BwdParams& p, const Tables& t, hipStream_t s) {
    return p.d == 64 ? launch_bwd_d<64>(p, t, s) : launch_bwd_d<128>(p, t, s);
}

}  // namespace wpa

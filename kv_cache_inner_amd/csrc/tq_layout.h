// Compile-time description of a packed-key layout and of the scorer's operand plan.
//
// Stored words (the bank format, see include/tq.h): per key, for each channel group g
// the b_g bit-planes of the bucket indices (d_g/32 words each), then m/32 sign words.
//
// The scorer never decodes a bucket index into a centroid. For a symmetric codebook
// (c[L-1-i] = -c[i], which Lloyd-Max for N(0,1) gives) the centroid is an odd function
// of the index bits in +-1 form, s_p = 2*b_p - 1, so it expands exactly over the odd
// subsets S of the bits (a Walsh expansion):
//     c[idx] = sum_{S odd} chat_S * prod_{p in S} s_p,
// 1 bit: {0}; 2 bits: {0},{1}; 3 bits: {0},{1},{2},{0,1,2}. Each product is 2*beta_S - 1
// with beta_S the XOR of the bits in S (odd |S|). So <qR, c[idx]> is a sum of binary dot
// products <2 chat_S qR, beta_S> minus c[L-1] * sum(qR). The "derived words" below are the
// beta_S bit vectors (one per subset, d_g/32 words each) followed by the sign words.
//
// MFMA plan (v_mfma_i32_16x16x64_i8, one 64-deep K step = 4 lane groups x 16 bytes):
// derived words are taken in quads; in quad q lane group gl holds derived word 4q+gl and
// expands it twice (halves h = 0, 1) into 16 bytes, byte e of dword v being bit
// (8e + 4h + v) of the word scaled by 2^(4h+v). A quad whose four words belong to more
// than one estimator term ("class": group 0, group 1, sketch) is issued once per class,
// the other class's weights being zero.
#pragma once

namespace tq {

constexpr int walsh_planes(int b) { return b == 3 ? 4 : b; }
// bit mask of the s-th odd subset of {0..b-1}
constexpr int walsh_mask(int b, int s) { return (b == 3 && s == 3) ? 7 : (1 << s); }

struct DWord {
    int cls;   // 0/1: codebook group, NG: sketch, -1: padding
    int nx;    // number of stored words XORed
    int s[3];  // stored word indices
    int sub;   // Walsh subset index within the group (codebook classes)
    int k;     // word index inside its plane (bit t of the word = element 32k+t)
};

template <int NG_, int D0_, int B0_, int D1_, int B1_, int M_>
struct Layout {
    static constexpr int NG = NG_;
    static constexpr int D0 = D0_, B0 = B0_;
    static constexpr int D1 = NG_ > 1 ? D1_ : 0, B1 = NG_ > 1 ? B1_ : 0;
    static constexpr int M = M_;
    static constexpr int D = D0 + D1;
    // the bank's norms: float32 here, binary16 in HalfNorms<Layout>
    static constexpr bool NH = false;
    using NormT = float;
    static constexpr int NCLS = NG + 1;
    static constexpr int SWG0 = B0 * D0 / 32, SWG1 = B1 * D1 / 32, SWS = M / 32;
    static constexpr int W = SWG0 + SWG1 + SWS;  // stored words per key
    static constexpr int NSQ = (W + 3) / 4;      // stored quads
    static constexpr int DWG0 = walsh_planes(B0) * D0 / 32;
    static constexpr int DWG1 = NG > 1 ? walsh_planes(B1) * D1 / 32 : 0;
    static constexpr int DW = DWG0 + DWG1 + SWS;  // derived words per key
    static constexpr int NQ = (DW + 3) / 4;       // derived quads (MFMA K-steps x 2)

    static_assert(D0 % 32 == 0 && D1 % 32 == 0 && M % 32 == 0 && M > 0, "dims must be multiples of 32");
    static_assert(B0 >= 1 && B0 <= 3 && (NG == 1 || (B1 >= 1 && B1 <= 3)), "codebook bits 1..3");

    static constexpr DWord dword(int dw) {
        DWord r{-1, 0, {0, 0, 0}, 0, 0};
        if (dw < DWG0) {
            const int wpp = D0 / 32;
            r.cls = 0;
            r.sub = dw / wpp;
            r.k = dw % wpp;
            const int mask = walsh_mask(B0, r.sub);
            for (int p = 0; p < B0; ++p)
                if (mask & (1 << p)) r.s[r.nx++] = p * wpp + r.k;
        } else if (dw < DWG0 + DWG1) {
            const int wpp = D1 > 0 ? D1 / 32 : 1, loc = dw - DWG0;
            r.cls = 1;
            r.sub = loc / wpp;
            r.k = loc % wpp;
            const int mask = walsh_mask(B1, r.sub);
            for (int p = 0; p < B1; ++p)
                if (mask & (1 << p)) r.s[r.nx++] = SWG0 + p * wpp + r.k;
        } else if (dw < DW) {
            r.cls = NG;
            r.k = dw - DWG0 - DWG1;
            r.nx = 1;
            r.s[0] = SWG0 + SWG1 + r.k;
        }
        return r;
    }

    // number of XOR components of quad q (max over its lane groups)
    static constexpr int quad_nx(int q) {
        int n = 0;
        for (int g = 0; g < 4; ++g) {
            const DWord w = dword(4 * q + g);
            if (w.cls >= 0 && w.nx > n) n = w.nx;
        }
        return n;
    }
    // stored quad index of component c of quad q (lane group gl reads stored word 4*sq+gl)
    static constexpr int quad_sq(int q, int c) {
        for (int g = 0; g < 4; ++g) {
            const DWord w = dword(4 * q + g);
            if (w.cls >= 0) return (w.s[c] - g) / 4;
        }
        return 0;
    }
    static constexpr bool quad_uniform(int q) {
        const int nx = quad_nx(q);
        for (int g = 0; g < 4; ++g) {
            const DWord w = dword(4 * q + g);
            if (w.cls < 0) continue;
            if (w.nx != nx) return false;
            for (int c = 0; c < nx; ++c)
                if (w.s[c] - g < 0 || (w.s[c] - g) % 4 != 0 || (w.s[c] - g) / 4 != quad_sq(q, c)) return false;
        }
        return true;
    }
    static constexpr bool all_uniform() {
        for (int q = 0; q < NQ; ++q)
            if (!quad_uniform(q)) return false;
        return true;
    }
    static_assert(all_uniform(), "layout needs codebook planes with XOR subsets aligned to 128 channels");

    static constexpr bool quad_has(int q, int c) {
        for (int g = 0; g < 4; ++g)
            if (dword(4 * q + g).cls == c) return true;
        return false;
    }
    // fragments enumerate (q, h, c) with c present in quad q
    static constexpr int frag_index(int q, int h, int c) {
        int f = 0;
        for (int qq = 0; qq < NQ; ++qq)
            for (int hh = 0; hh < 2; ++hh)
                for (int cc = 0; cc < NCLS; ++cc)
                    if (quad_has(qq, cc)) {
                        if (qq == q && hh == h && cc == c) return f;
                        ++f;
                    }
        return -1;
    }
    static constexpr int count_frags() {
        int f = 0;
        for (int q = 0; q < NQ; ++q)
            for (int c = 0; c < NCLS; ++c) f += quad_has(q, c) ? 2 : 0;
        return f;
    }
    static constexpr int NF = count_frags();

    // bit positions feeding estimator term c (bounds its integer limb sums)
    static constexpr int class_positions(int c) {
        int n = 0;
        for (int dw = 0; dw < DW; ++dw)
            if (dword(dw).cls == c) n += 32;
        return n;
    }

    // inverse of frag_index: quad, half and class of fragment f
    static constexpr int frag_field(int f, int which) {
        int k = 0;
        for (int q = 0; q < NQ; ++q)
            for (int h = 0; h < 2; ++h)
                for (int c = 0; c < NCLS; ++c)
                    if (quad_has(q, c)) {
                        if (k == f) return which == 0 ? q : which == 1 ? h : c;
                        ++k;
                    }
        return -1;
    }
    static constexpr int frag_q(int f) { return frag_field(f, 0); }
    static constexpr int frag_h(int f) { return frag_field(f, 1); }
    static constexpr int frag_c(int f) { return frag_field(f, 2); }
};

// The same layout with its bank's norms stored as binary16 (the 16-bit norm format).
template <class L>
struct HalfNorms : L {
    static constexpr bool NH = true;
    using NormT = uint16_t;
};

}  // namespace tq

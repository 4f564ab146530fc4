// pq_selftest: known-answer checks of every entry point on tiny inputs whose
// results follow in closed form (no reference implementation involved):
//  - q8 of blocks whose max |x| is 127 (scale exactly 1, so q = round(x));
//  - routing of increasing / decreasing logits (ids known; softmax weights
//    e^-j / sum_i e^-i);
//  - grouping of the resulting id list (offsets, order and active list known);
//  - ternary and grid1 mat-vecs and the prefill GEMM with every weight +1 and
//    unit scales: each output is the exact integer sum of its activations;
//  - the fused prep against the same answers; combine and fused combine with
//    known weights; validation of a plane with a known number of code-3 fields.
// Allocates device memory and synchronizes the stream (not a hot-path call).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "../../include/pq.h"

namespace {

struct DevBuf {
    void* p = nullptr;
    size_t n = 0;
    DevBuf() = default;
    DevBuf(const DevBuf&) = delete;
    DevBuf& operator=(const DevBuf&) = delete;
    ~DevBuf() {
        if (p) (void)hipFree(p);
    }
    bool alloc(size_t bytes) {
        n = bytes;
        return hipMalloc(&p, bytes) == hipSuccess;
    }
    template <typename T>
    bool put(const std::vector<T>& h) {
        return alloc(h.size() * sizeof(T)) &&
               hipMemcpy(p, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice) == hipSuccess;
    }
    template <typename T>
    bool get(std::vector<T>& h) const {
        return hipMemcpy(h.data(), p, h.size() * sizeof(T), hipMemcpyDeviceToHost) == hipSuccess;
    }
    template <typename T>
    T* as() const {
        return static_cast<T*>(p);
    }
};

struct Fail {};

constexpr int kT = 2, kE = 8, kK = 4, kA = kT * kK;
constexpr int kH = 256, kRows = 32;   // matrix [kRows][kH]
constexpr uint16_t kHalfOne = 0x3C00;  // fp16 1.0

void ok(bool c) {
    if (!c) throw Fail{};
}
void hip_ok(hipError_t e) {
    if (e != hipSuccess) throw e;
}
void pq_ok(pq_status s) {
    if (s == PQ_ERR_HIP) throw hipErrorUnknown;
    ok(s == PQ_OK);
}

// Activation row t: every 32-block holds +127 at its first element (so the q8
// scale is exactly 1) and small integers elsewhere.
float act_value(int t, int c) {
    if (c % 32 == 0) return 127.0f;
    return static_cast<float>((c * 37 + t * 11) % 101 - 50);
}

pq_status run(hipStream_t s) {
    pq_stream st = s;
    // ---- q8 of hand-picked blocks
    {
        std::vector<float> x(64, 0.0f);
        const float v[8] = {127.0f, -127.0f, 2.5f, -2.5f, 0.5f, -0.49f, 126.5f, 1.0f};
        const int8_t q[8] = {127, -127, 3, -3, 1, 0, 127, 1};
        for (int i = 0; i < 8; ++i) x[i] = v[i];
        DevBuf dx, dq, dd;
        ok(dx.put(x) && dq.alloc(64) && dd.alloc(2 * sizeof(float)));
        pq_ok(pq_quantize_act_q8(dx.as<float>(), 1, 64, dq.as<int8_t>(), dd.as<float>(), st));
        hip_ok(hipStreamSynchronize(s));
        std::vector<int8_t> hq(64);
        std::vector<float> hd(2);
        ok(dq.get(hq) && dd.get(hd));
        for (int i = 0; i < 64; ++i) ok(hq[i] == (i < 8 ? q[i] : 0));
        ok(hd[0] == 1.0f && hd[1] == 0.0f);
    }

    // ---- routing, grouping, prep
    std::vector<float> logits(kT * kE), x(kT * kH);
    for (int e = 0; e < kE; ++e) {
        logits[e] = static_cast<float>(e);
        logits[kE + e] = static_cast<float>(kE - 1 - e);
    }
    for (int t = 0; t < kT; ++t)
        for (int c = 0; c < kH; ++c) x[t * kH + c] = act_value(t, c);
    const int32_t ids_ref[kA] = {7, 6, 5, 4, 0, 1, 2, 3};
    const int32_t sorted_ref[kA] = {4, 5, 6, 7, 3, 2, 1, 0};
    double wden = 0.0;
    for (int j = 0; j < kK; ++j) wden += std::exp(-static_cast<double>(j));
    DevBuf dlog, dx, dids, dw, doff, dsorted, dact, dnact, dxq, dxd;
    ok(dlog.put(logits) && dx.put(x) && dids.alloc(kA * 4) && dw.alloc(kA * 4) &&
       doff.alloc((kE + 1) * 4) && dsorted.alloc(kA * 4) && dact.alloc(kE * 4) && dnact.alloc(4) &&
       dxq.alloc(kT * kH) && dxd.alloc(kT * kH / 32 * 4));
    auto check_routing = [&]() {
        hip_ok(hipStreamSynchronize(s));
        std::vector<int32_t> ids(kA), off(kE + 1), srt(kA), act(kE), na(1);
        std::vector<float> w(kA), xd(kT * kH / 32);
        std::vector<int8_t> xq(kT * kH);
        ok(dids.get(ids) && dw.get(w) && doff.get(off) && dsorted.get(srt) && dact.get(act) &&
           dnact.get(na) && dxq.get(xq) && dxd.get(xd));
        for (int a = 0; a < kA; ++a) {
            ok(ids[a] == ids_ref[a] && srt[a] == sorted_ref[a]);
            const double wr = std::exp(-static_cast<double>(a % kK)) / wden;
            ok(std::fabs(w[a] - wr) <= 1e-6);
        }
        for (int e = 0; e <= kE; ++e) ok(off[e] == e);
        ok(na[0] == kE);
        for (int e = 0; e < kE; ++e) ok(act[e] == e);
        for (int i = 0; i < kT * kH; ++i) ok(xq[i] == static_cast<int8_t>(x[i]));
        for (float d : xd) ok(d == 1.0f);
    };
    pq_ok(pq_quantize_act_q8(dx.as<float>(), kT, kH, dxq.as<int8_t>(), dxd.as<float>(), st));
    pq_ok(pq_moe_route_topk(dlog.as<float>(), kT, kE, kK, dids.as<int32_t>(), dw.as<float>(), st));
    pq_ok(pq_group_tokens_by_expert(dids.as<int32_t>(), kT, kK, kE, doff.as<int32_t>(),
                                    dsorted.as<int32_t>(), dact.as<int32_t>(), dnact.as<int32_t>(), st));
    check_routing();
    hip_ok(hipMemsetAsync(dids.p, 0xff, kA * 4, s));
    hip_ok(hipMemsetAsync(dsorted.p, 0xff, kA * 4, s));
    hip_ok(hipMemsetAsync(dxq.p, 0, kT * kH, s));
    pq_ok(pq_moe_decode_prep(dx.as<float>(), dlog.as<float>(), kT, kH, kE, kK, dxq.as<int8_t>(),
                             dxd.as<float>(), dids.as<int32_t>(), dw.as<float>(), doff.as<int32_t>(),
                             dsorted.as<int32_t>(), dact.as<int32_t>(), dnact.as<int32_t>(), nullptr, st));
    check_routing();
    const pq_groups g{doff.as<int32_t>(), dsorted.as<int32_t>(), dact.as<int32_t>(), dnact.as<int32_t>(),
                      kT, kK, kE};

    // exact row sums of the activations of token t
    double sum_t[kT] = {0.0, 0.0};
    for (int t = 0; t < kT; ++t)
        for (int c = 0; c < kH; ++c) sum_t[t] += x[t * kH + c];

    // ---- all-(+1) weights with unit scales
    std::vector<uint8_t> tq(static_cast<size_t>(kE) * kRows * kH / 4, 0x55);   // four codes 1
    std::vector<uint16_t> dsc(static_cast<size_t>(kE) * kRows * kH / 256, kHalfOne);
    std::vector<uint8_t> gqs(static_cast<size_t>(kE) * kRows * kH / 8);
    std::vector<uint16_t> gqh(static_cast<size_t>(kE) * kRows * kH / 32);
    for (size_t i = 0; i < gqs.size(); ++i) gqs[i] = static_cast<uint8_t>(i * 29 + 3);
    for (size_t i = 0; i < gqh.size(); ++i) gqh[i] = static_cast<uint16_t>((i * 1237 + 11) & 0x0fff);
    std::vector<int8_t> grid(2048 * 8, 1);
    DevBuf dtq, dsc_d, dgqs, dgqh, dgrid, dout, dy;
    ok(dtq.put(tq) && dsc_d.put(dsc) && dgqs.put(gqs) && dgqh.put(gqh) && dgrid.put(grid) &&
       dout.alloc(kA * kRows * 4) && dy.alloc(kT * kRows * 4));
    auto check_out = [&]() {
        hip_ok(hipStreamSynchronize(s));
        std::vector<float> out(kA * kRows);
        ok(dout.get(out));
        for (int a = 0; a < kA; ++a)
            for (int n = 0; n < kRows; ++n) ok(out[a * kRows + n] == static_cast<float>(sum_t[a / kK]));
    };
    const pq_ternary_w tw{dtq.as<uint8_t>(), dsc_d.as<uint16_t>(), kE, kRows, kH};
    hip_ok(hipMemsetAsync(dout.p, 0, dout.n, s));
    pq_ok(pq_moe_matvec_ternary(&tw, nullptr, &g, dxq.as<int8_t>(), dxd.as<float>(), 1, PQ_EPI_F32,
                                dout.p, nullptr, nullptr, st));
    check_out();
    const pq_grid1_w gw{dgqs.as<uint8_t>(), dgqh.as<uint16_t>(), dsc_d.as<uint16_t>(), dgrid.as<int8_t>(),
                        kE, kRows, kH};
    hip_ok(hipMemsetAsync(dout.p, 0, dout.n, s));
    pq_ok(pq_moe_matvec_grid1(&gw, nullptr, &g, dxq.as<int8_t>(), dxd.as<float>(), 1, PQ_EPI_F32,
                              dout.p, nullptr, nullptr, st));
    check_out();
    {
        std::vector<uint16_t> xb(kT * kH);   // integers |v| <= 127 are exact in bf16
        for (int i = 0; i < kT * kH; ++i) {
            uint32_t u;
            std::memcpy(&u, &x[i], 4);
            xb[i] = static_cast<uint16_t>(u >> 16);
        }
        DevBuf dxb, dtqs, dtqh;
        ok(dxb.put(xb) && dtqs.alloc(dgqs.n) && dtqh.alloc(dgqh.n));
        pq_ok(pq_tile_layout_grid1(&gw, dtqs.as<uint8_t>(), dtqh.as<uint16_t>(), st));
        const pq_grid1_w gwt{dtqs.as<uint8_t>(), dtqh.as<uint16_t>(), dsc_d.as<uint16_t>(), dgrid.as<int8_t>(),
                             kE, kRows, kH};
        hip_ok(hipMemsetAsync(dout.p, 0, dout.n, s));
        pq_ok(pq_moe_gemm_dequant_tile(&gwt, nullptr, &g, dxb.as<uint16_t>(), 1, PQ_EPI_F32, dout.p,
                                       nullptr, nullptr, st));
        check_out();
    }
    // ---- sub-scaled signs: every sign positive, every sub-scale 1, anchors 1
    std::vector<uint8_t> ssg(static_cast<size_t>(kE) * kRows * kH / 8, 0);
    std::vector<uint8_t> ssc(static_cast<size_t>(kE) * kRows * kH / 32, 0x11);
    std::vector<uint16_t> sanc(static_cast<size_t>(kE) * kRows, kHalfOne);
    DevBuf dssg, dssc, dsanc;
    ok(dssg.put(ssg) && dssc.put(ssc) && dsanc.put(sanc));
    const pq_sign1_w sw{dssg.as<uint8_t>(), dssc.as<uint8_t>(), dsanc.as<uint16_t>(), kE, kRows, kH};
    hip_ok(hipMemsetAsync(dout.p, 0, dout.n, s));
    pq_ok(pq_moe_matvec_sign1(&sw, nullptr, &g, dxq.as<int8_t>(), dxd.as<float>(), 1, PQ_EPI_F32,
                              dout.p, nullptr, nullptr, st));
    check_out();
    // ---- sub-scaled signs in the prefill GEMM (hidden 512: whole 16-byte
    // sub-scale units), bf16 activations that are small integers (exact)
    {
        constexpr int kH2 = 512;
        std::vector<uint16_t> xb2(kT * kH2);
        double s2[kT] = {0.0, 0.0};
        for (int t = 0; t < kT; ++t)
            for (int c = 0; c < kH2; ++c) {
                const float v = static_cast<float>((t * 7 + c * 3) % 17 - 8);
                uint32_t u;
                std::memcpy(&u, &v, 4);
                xb2[t * kH2 + c] = static_cast<uint16_t>(u >> 16);
                s2[t] += v;
            }
        std::vector<uint8_t> sg2(static_cast<size_t>(kE) * kRows * kH2 / 8, 0);
        std::vector<uint8_t> sc2(static_cast<size_t>(kE) * kRows * kH2 / 32, 0x11);
        DevBuf dxb2, dsg2, dsc2, dtsg, dtsc;
        ok(dxb2.put(xb2) && dsg2.put(sg2) && dsc2.put(sc2) && dtsg.alloc(dsg2.n) && dtsc.alloc(dsc2.n));
        const pq_sign1_w sw2{dsg2.as<uint8_t>(), dsc2.as<uint8_t>(), dsanc.as<uint16_t>(), kE, kRows, kH2};
        pq_ok(pq_tile_layout_sign1(&sw2, dtsg.as<uint8_t>(), dtsc.as<uint8_t>(), st));
        const pq_sign1_w sw2t{dtsg.as<uint8_t>(), dtsc.as<uint8_t>(), dsanc.as<uint16_t>(), kE, kRows, kH2};
        hip_ok(hipMemsetAsync(dout.p, 0, dout.n, s));
        pq_ok(pq_moe_gemm_dequant_tile_sign1(&sw2t, nullptr, &g, dxb2.as<uint16_t>(), 1, PQ_EPI_F32, dout.p,
                                             nullptr, nullptr, st));
        hip_ok(hipStreamSynchronize(s));
        std::vector<float> out(kA * kRows);
        ok(dout.get(out));
        for (int a = 0; a < kA; ++a)
            for (int n = 0; n < kRows; ++n) ok(out[a * kRows + n] == static_cast<float>(s2[a / kK]));
    }
    // ---- the int8-MFMA tile in all three formats (same answers)
    hip_ok(hipMemsetAsync(dout.p, 0, dout.n, s));
    pq_ok(pq_moe_tile_q8_ternary(&tw, nullptr, &g, dxq.as<int8_t>(), dxd.as<float>(), 1, PQ_EPI_F32,
                                 dout.p, nullptr, nullptr, st));
    check_out();
    hip_ok(hipMemsetAsync(dout.p, 0, dout.n, s));
    pq_ok(pq_moe_tile_q8_grid1(&gw, nullptr, &g, dxq.as<int8_t>(), dxd.as<float>(), 1, PQ_EPI_F32,
                               dout.p, nullptr, nullptr, st));
    check_out();
    hip_ok(hipMemsetAsync(dout.p, 0, dout.n, s));
    pq_ok(pq_moe_tile_q8_sign1(&sw, nullptr, &g, dxq.as<int8_t>(), dxd.as<float>(), 1, PQ_EPI_F32,
                               dout.p, nullptr, nullptr, st));
    check_out();

    // ---- combine: separate (out = the exact sums above), and fused into the
    // mat-vec (activation row = assignment: use the q8 rows of token a/k)
    pq_ok(pq_moe_combine(dout.as<float>(), dw.as<float>(), kT, kK, kRows, dy.as<float>(), st));
    auto check_y = [&]() {
        hip_ok(hipStreamSynchronize(s));
        std::vector<float> y(kT * kRows);
        ok(dy.get(y));
        for (int t = 0; t < kT; ++t)
            for (int n = 0; n < kRows; ++n)
                ok(std::fabs(y[t * kRows + n] - sum_t[t]) <= 1e-5 * std::fabs(sum_t[t]) + 1e-6);
    };
    check_y();
    {
        std::vector<int8_t> xq_a(kA * kH);
        std::vector<float> xd_a(kA * kH / 32, 1.0f);
        for (int a = 0; a < kA; ++a)
            for (int c = 0; c < kH; ++c) xq_a[a * kH + c] = static_cast<int8_t>(x[(a / kK) * kH + c]);
        DevBuf dxqa, dxda;
        ok(dxqa.put(xq_a) && dxda.put(xd_a));
        hip_ok(hipMemsetAsync(dy.p, 0, dy.n, s));
        pq_ok(pq_moe_matvec_ternary(&tw, nullptr, &g, dxqa.as<int8_t>(), dxda.as<float>(), 0,
                                    PQ_EPI_F32_COMBINE, dy.p, dw.p, nullptr, st));
        check_y();
    }

    // ---- validation: 3 bytes 0xFF (4 code-3 fields each) and 1 byte 0x0F
    // (2) in an otherwise valid plane
    {
        std::vector<uint8_t> bad(tq);
        bad[5] = 0xff;
        bad[700] = 0xff;
        bad[bad.size() - 1] = 0xff;
        bad[33] = 0x0f;
        DevBuf dbad, dn;
        ok(dbad.put(bad) && dn.alloc(4));
        const pq_ternary_w bw{dbad.as<uint8_t>(), dsc_d.as<uint16_t>(), kE, kRows, kH};
        pq_ok(pq_validate_ternary(&bw, dn.as<int32_t>(), st));
        hip_ok(hipStreamSynchronize(s));
        std::vector<int32_t> n(1);
        ok(dn.get(n));
        ok(n[0] == 14);
    }
    return PQ_OK;
}

}  // namespace

extern "C" pq_status pq_selftest(pq_stream stream) {
    try {
        return run(static_cast<hipStream_t>(stream));
    } catch (Fail&) {
        return PQ_ERR_SELFTEST;
    } catch (hipError_t&) {
        return PQ_ERR_HIP;
    } catch (...) {
        return PQ_ERR_HIP;
    }
}

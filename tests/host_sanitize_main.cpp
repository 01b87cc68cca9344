// Host code under AddressSanitizer and UndefinedBehaviorSanitizer: the CPU
// oracle (oracle/oracle.c) and the plan code (tp_plan.cpp) are driven over
// small and benchmark-sized shapes, valid and invalid, and this program
// exits 0 only if every call returned what it should. The sanitizers abort
// the run on the first out-of-bounds access, use after free, signed
// overflow or other undefined behaviour they see. Test infrastructure: built
// and run by tests/test_host_sanitize.py with g++ only (no device code).
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "tp_decode.h"

extern "C" {
uint16_t oracle_f32_to_bf16(float f);
void oracle_partial(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t batch, int64_t k,
                    int64_t hidden, double* y64, float* y32, int nthreads);
int oracle_ring_reduce(const float* partials, int32_t n_ranks, int64_t len, const float* residual,
                       float* out, uint16_t* out_bf16);
int64_t oracle_ring_wire_bytes_per_rank(int32_t n_ranks, int64_t payload_elems, int32_t elem_bytes);
int oracle_decode_layers(int32_t n_layers, int32_t n_ranks, int32_t rank, int64_t batch, int64_t hidden,
                         int64_t ka_r, int64_t ki_r, const uint16_t* x_attn, const uint16_t* w_o,
                         const uint16_t* x_ffn, const uint16_t* w_down, float* slots, float* hidden_state,
                         int nthreads);
int oracle_moe_route(const float* logits, int32_t tokens, int32_t experts, int32_t top_k, int32_t renorm,
                     int32_t* sel_expert, double* sel_weight);
int oracle_gate_up_swiglu(const uint16_t* x, const uint16_t* w_gate, const uint16_t* w_up, int64_t batch,
                          int64_t hidden, int64_t cols, double* a64, uint16_t* a_bf16, int nthreads);
int oracle_qkv_proj(const uint16_t* x, const uint16_t* w, int64_t batch, int64_t hidden, int64_t cols,
                    double* a64, uint16_t* a_bf16, int nthreads);
int oracle_mx_quantize(int32_t fmt, const uint16_t* w, int64_t K, int64_t H, uint8_t* codes,
                       uint8_t* scales);
int oracle_mx_partial(int32_t fmt, const uint16_t* x, int64_t batch, int64_t K, int64_t H,
                      const uint8_t* codes, const uint8_t* scales, double* y64, float* y32, int nthreads);
}

static int failures = 0;
#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

// xorshift64* values in about [-1, 1)
static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static float next_f() {
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (float)((rng_state * 0x2545f4914f6cdd1dull) >> 40) / (float)(1u << 23) - 1.0f;
}
static std::vector<uint16_t> bf16_vec(size_t n, float scale) {
    std::vector<uint16_t> v(n);
    for (auto& e : v) e = oracle_f32_to_bf16(scale * next_f());
    return v;
}
static std::vector<float> f32_vec(size_t n) {
    std::vector<float> v(n);
    for (auto& e : v) e = next_f();
    return v;
}

static void oracle_cases() {
    // projection partials, one and several threads, ragged sizes
    const int64_t shapes[][3] = {{1, 1, 1}, {3, 17, 40}, {5, 64, 129}, {2, 130, 8}};
    for (auto& s : shapes) {
        const int64_t b = s[0], k = s[1], h = s[2];
        auto x = bf16_vec(b * k, 1.f);
        auto w = bf16_vec(k * h, 0.02f);
        for (int t : {1, 3}) {
            std::vector<double> y64(b * h);
            std::vector<float> y32(b * h);
            oracle_partial(x.data(), k, w.data(), b, k, h, y64.data(), y32.data(), t);
        }
    }
    // ring-order sum, every rank count, with and without the bf16 output
    for (int n = 1; n <= 8; ++n) {
        const int64_t len = 6 * n;
        auto p = f32_vec(n * len);
        auto r = f32_vec(len);
        std::vector<float> out(len);
        std::vector<uint16_t> ob(len);
        EXPECT(oracle_ring_reduce(p.data(), n, len, r.data(), out.data(), ob.data()) == 0);
        EXPECT(oracle_ring_reduce(p.data(), n, len, r.data(), out.data(), nullptr) == 0);
        EXPECT(oracle_ring_wire_bytes_per_rank(n, len, 2) == (int64_t)2 * (n - 1) * (len / n) * 2);
    }
    EXPECT(oracle_ring_reduce(nullptr, 3, 7, nullptr, nullptr, nullptr) != 0);  // N must divide len
    // the decode step over a small stack, every rank
    {
        const int L = 2, n = 3, b = 2;
        const int64_t h = 24, ka = 12, ki = 30, kar = ka / n, kir = ki / n;
        auto xa = bf16_vec((size_t)L * b * kar, 1.f), wo = bf16_vec((size_t)L * kar * h, 0.02f);
        auto xf = bf16_vec((size_t)L * b * kir, 1.f), wd = bf16_vec((size_t)L * kir * h, 0.02f);
        for (int rank = 0; rank < n; ++rank) {
            auto slots = f32_vec((size_t)L * 2 * n * b * h);
            auto hs = f32_vec((size_t)b * h);
            EXPECT(oracle_decode_layers(L, n, rank, b, h, kar, kir, xa.data(), wo.data(), xf.data(),
                                        wd.data(), slots.data(), hs.data(), 2) == 0);
        }
    }
    // routing: softmax, top-k, renormalised or not
    {
        const int T = 5, E = 16, K = 4;
        auto lg = f32_vec(T * E);
        std::vector<int32_t> se(T * K);
        std::vector<double> sw(T * K);
        EXPECT(oracle_moe_route(lg.data(), T, E, K, 1, se.data(), sw.data()) == 0);
        EXPECT(oracle_moe_route(lg.data(), T, E, K, 0, se.data(), sw.data()) == 0);
        for (int i = 0; i < T * K; ++i) EXPECT(se[i] >= 0 && se[i] < E);
        EXPECT(oracle_moe_route(lg.data(), T, E, E + 1, 1, se.data(), sw.data()) != 0);
    }
    // column-parallel up projection with SwiGLU, and the QKV projection
    {
        const int64_t b = 3, h = 40, c = 24;
        auto x = bf16_vec(b * h, 1.f), wg = bf16_vec(h * c, 0.02f), wu = bf16_vec(h * c, 0.02f);
        std::vector<double> a64(b * c);
        std::vector<uint16_t> ab(b * c);
        EXPECT(oracle_gate_up_swiglu(x.data(), wg.data(), wu.data(), b, h, c, a64.data(), ab.data(), 2) == 0);
        EXPECT(oracle_qkv_proj(x.data(), wg.data(), b, h, c, a64.data(), ab.data(), 2) == 0);
    }
    // microscaled weights: quantisation and projection, both formats
    for (int fmt : {1, 2}) {
        const int64_t K = 64, H = 12, b = 2;
        auto w = bf16_vec(K * H, 0.02f);
        auto x = bf16_vec(b * K, 1.f);
        std::vector<uint8_t> codes(K * H), scales(K / 32 * H);
        EXPECT(oracle_mx_quantize(fmt, w.data(), K, H, codes.data(), scales.data()) == 0);
        std::vector<double> y64(b * H);
        std::vector<float> y32(b * H);
        EXPECT(oracle_mx_partial(fmt, x.data(), b, K, H, codes.data(), scales.data(), y64.data(), y32.data(),
                                 2) == 0);
        EXPECT(oracle_mx_quantize(fmt, w.data(), 48, H, codes.data(), scales.data()) != 0);  // K % 32
    }
}

static void plan_cases() {
    // (H, I, N, b, k_attn, qkv columns): tiny, the benchmarked stacks, odd sizes
    const int64_t shapes[][6] = {
        {512, 1376, 2, 1, 0, 0},      {5120, 17408, 4, 1, 0, 1536}, {5120, 17408, 2, 32, 0, 3072},
        {4096, 12288, 8, 64, 0, 768}, {4096, 12288, 4, 16, 8192, 0}, {1032, 2048, 4, 3, 640, 0},
        {24, 48, 3, 4, 24, 0},        {16400, 256, 2, 1, 128, 0},   {64, 128, 1, 64, 0, 8}};
    const char* knobs[][2] = {{"serial_points", "1"}, {"segment_loads", "4"}, {"stream_kind", "1"},
                              {"stream_kind", "2"},   {"valu_cols", "256"},   {"splits_ffn", "4"},
                              {"mfma_flat", "1"},     {"xcd_walk", "1"}};
    for (auto& s : shapes) {
        for (int variant = 0; variant < 4; ++variant) {
            tp_plan_t p = nullptr;
            if (tp_plan(s[0], s[1], (int32_t)s[2], (int32_t)s[3], &p) != TP_OK) {
                ++failures;
                fprintf(stderr, "tp_plan failed for H=%lld\n", (long long)s[0]);
                continue;
            }
            if (s[4]) EXPECT(tp_plan_set_attn_dim(p, s[4]) == TP_OK);
            if (s[5]) EXPECT(tp_plan_set_qkv_dim(p, s[5]) == TP_OK);
            if (variant == 1) tp_plan_set_weight_format(p, TP_WEIGHTS_MXFP8);  // may be refused
            if (variant == 2) tp_plan_set_weight_format(p, TP_WEIGHTS_MXFP4);
            if (variant == 3)
                for (auto& kv : knobs) tp_plan_tune(p, kv[0], atoll(kv[1]));  // may be refused
            struct tp_plan_info info;
            memset(&info, 0, sizeof info);
            EXPECT(tp_plan_info(p, &info) == TP_OK);
            EXPECT(info.hidden == s[0] && info.n_ranks == s[2] && info.workspace_bytes > 0);
            EXPECT(tp_plan_info_get(p, &info) == TP_OK);
            tp_plan_destroy(p);
        }
    }
    // the MoE share
    {
        tp_plan_t p = nullptr;
        EXPECT(tp_plan(4096, 12288, 4, 64, &p) == TP_OK);
        EXPECT(tp_plan_set_attn_dim(p, 8192) == TP_OK);
        EXPECT(tp_plan_set_moe(p, 128, 8, 4, 1536, 64) == TP_OK);
        struct tp_plan_info info;
        EXPECT(tp_plan_info(p, &info) == TP_OK && info.local_experts == 32);
        EXPECT(tp_plan_set_moe(p, 128, 129, 4, 1536, 64) != TP_OK);
        tp_plan_destroy(p);
    }
    // invalid plans and knobs
    tp_plan_t p = nullptr;
    EXPECT(tp_plan(0, 128, 2, 1, &p) != TP_OK);
    EXPECT(tp_plan(512, 1376, 3, 1, &p) != TP_OK);
    EXPECT(tp_plan(512, 1376, 2, 65, &p) != TP_OK);
    EXPECT(tp_plan(512, 1376, 2, 1, &p) == TP_OK);
    EXPECT(tp_plan_tune(p, "no_such_knob", 1) != TP_OK);
    EXPECT(tp_plan_set_attn_dim(p, 7) != TP_OK);
    EXPECT(tp_plan_set_qkv_dim(p, 12) != TP_OK);
    EXPECT(tp_status_str(TP_ERR_INVALID_ARG) != nullptr);
    tp_plan_destroy(p);
}

int main() {
    oracle_cases();
    plan_cases();
    if (failures) {
        fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("host sanitizer run: ok\n");
    return 0;
}

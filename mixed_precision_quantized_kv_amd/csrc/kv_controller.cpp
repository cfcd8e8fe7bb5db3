// kv_controller.cpp -- the EchoKV bit-width controller (host): canary readings in, one width per
// layer out.
//
// EchoKV, "Show the math -- what the canary actually computes": each firing yields one KL
// reading per (layer, width b in {2, 4, 8}); each reading is smoothed by its own exponential
// moving average (alpha = 0.1), and a layer's width is the least b whose average is below the
// budget tau. The choice is taken again from scratch at every firing, so a layer can move up or
// down ("Bidirectional adjustment"), and the budget grows with the context length as
// tau(L) = tau0 * sqrt(L / L0), tau0 = 0.022 at L0 = 4K ("The tau(L) scaling"). "Measurement
// protocol -- warmup, freeze, measure": a frozen controller takes no further updates. A width
// change reaches the cache through kv_alloc_set_layer_bits, which only routes blocks allocated
// later ("What happens to old blocks when a layer changes tier?").
//
// Where the page is silent: the first reading of a (layer, width) pair starts its average;
// when no width is under the budget the layer goes to INT8; before its first firing a layer
// keeps the width it was created with. The averages are kept in binary64 and every operation is
// a single IEEE operation (this file is compiled without floating-point contraction), so the
// result does not depend on the compiler.
#include <cmath>
#include <new>
#include <vector>

#include "kv_quant.h"
#include "kvq_host.hpp"

struct kv_controller {
    int layers = 0;
    double alpha = 0.1, tau0 = 0.022, l0 = 4096.0;
    std::vector<double> ema;            // [layers][3]
    std::vector<unsigned char> seen;    // [layers][3]: a reading has arrived
    std::vector<int> bits;              // [layers]
    bool frozen = false;
    int64_t firings = 0;
};

namespace {

constexpr int kWidths[3] = {2, 4, 8};

bool valid_bits(int b) { return b == 2 || b == 4 || b == 8 || b == 16; }

}  // namespace

extern "C" {

double kv_controller_tau(double tau0, double l0, double context_len) {
    if (!(tau0 > 0.0) || !(l0 > 0.0) || !(context_len > 0.0)) return NAN;
    return tau0 * std::sqrt(context_len / l0);
}

kv_status kv_controller_create(int num_layers, const int* initial_bits, double alpha, double tau0,
                               double l0, kv_controller** out) {
    if (!out || !initial_bits) return kvq::fail(KV_EINVAL, "NULL argument");
    if (num_layers <= 0) return kvq::fail(KV_EINVAL, "num_layers %d", num_layers);
    if (!(alpha > 0.0 && alpha <= 1.0)) return kvq::fail(KV_EINVAL, "alpha %g outside (0, 1]", alpha);
    if (!(tau0 > 0.0) || !std::isfinite(tau0)) return kvq::fail(KV_EINVAL, "tau0 %g", tau0);
    if (!(l0 > 0.0) || !std::isfinite(l0)) return kvq::fail(KV_EINVAL, "L0 %g", l0);
    for (int l = 0; l < num_layers; ++l)
        if (!valid_bits(initial_bits[l]))
            return kvq::fail(KV_EINVAL, "layer %d initial bits %d", l, initial_bits[l]);
    kv_controller* c = new (std::nothrow) kv_controller;
    if (!c) return kvq::fail(KV_EINVAL, "out of host memory");
    c->layers = num_layers;
    c->alpha = alpha;
    c->tau0 = tau0;
    c->l0 = l0;
    try {
        c->ema.assign(3 * (size_t)num_layers, 0.0);
        c->seen.assign(3 * (size_t)num_layers, 0);
        c->bits.assign(initial_bits, initial_bits + num_layers);
    } catch (const std::bad_alloc&) {
        delete c;
        return kvq::fail(KV_EINVAL, "out of host memory");
    }
    *out = c;
    return kvq::ok();
}

kv_status kv_controller_observe(kv_controller* c, const float* kl, double context_len,
                                int* bits_out) {
    if (!c || !kl) return kvq::fail(KV_EINVAL, "NULL argument");
    if (!(context_len > 0.0) || !std::isfinite(context_len))
        return kvq::fail(KV_EINVAL, "context length %g", context_len);
    for (int i = 0; i < 3 * c->layers; ++i)     // a reading is a KL divergence: finite, >= 0
        if (!(kl[i] >= 0.0f) || !std::isfinite(kl[i]))
            return kvq::fail(KV_EINVAL, "reading %d (layer %d, INT%d) is %g", i, i / 3,
                             kWidths[i % 3], (double)kl[i]);
    if (!c->frozen) {
        const double budget = kv_controller_tau(c->tau0, c->l0, context_len);
        const double keep = 1.0 - c->alpha;
        for (int l = 0; l < c->layers; ++l) {
            int choice = 8;
            for (int j = 0; j < 3; ++j) {
                const size_t i = 3 * (size_t)l + j;
                const double x = (double)kl[i];
                if (c->seen[i]) {
                    const double decayed = keep * c->ema[i];
                    const double added = c->alpha * x;
                    c->ema[i] = decayed + added;
                } else {
                    c->ema[i] = x;
                    c->seen[i] = 1;
                }
            }
            for (int j = 0; j < 3; ++j)
                if (c->ema[3 * (size_t)l + j] < budget) {
                    choice = kWidths[j];
                    break;
                }
            c->bits[l] = choice;
        }
        ++c->firings;
    }
    if (bits_out)
        for (int l = 0; l < c->layers; ++l) bits_out[l] = c->bits[l];
    return kvq::ok();
}

kv_status kv_controller_set_frozen(kv_controller* c, int frozen) {
    if (!c) return kvq::fail(KV_EINVAL, "controller is NULL");
    c->frozen = frozen != 0;
    return kvq::ok();
}

kv_status kv_controller_state(const kv_controller* c, double* ema, int* bits, int64_t* firings) {
    if (!c) return kvq::fail(KV_EINVAL, "controller is NULL");
    if (ema)
        for (size_t i = 0; i < c->ema.size(); ++i) ema[i] = c->seen[i] ? c->ema[i] : NAN;
    if (bits)
        for (int l = 0; l < c->layers; ++l) bits[l] = c->bits[l];
    if (firings) *firings = c->firings;
    return kvq::ok();
}

kv_status kv_controller_apply(const kv_controller* c, kv_alloc* a) {
    if (!c || !a) return kvq::fail(KV_EINVAL, "NULL argument");
    // all-or-nothing: the layer counts must agree and every width must be one the allocator
    // routes, before any layer changes
    if (kv_alloc_layer_bits(a, c->layers - 1) == 0 || kv_alloc_layer_bits(a, c->layers) != 0)
        return kvq::fail(KV_EINVAL, "the allocator does not have %d layers", c->layers);
    for (int l = 0; l < c->layers; ++l)
        if (!kvq::alloc_accepts_bits(c->bits[l]))
            return kvq::fail(KV_EUNSUPPORTED, "layer %d: width %d has no pool", l, c->bits[l]);
    for (int l = 0; l < c->layers; ++l) {
        const kv_status st = kv_alloc_set_layer_bits(a, l, c->bits[l]);
        if (st != KV_OK) return st;
    }
    return kvq::ok();
}

void kv_controller_destroy(kv_controller* c) { delete c; }

}  // extern "C"

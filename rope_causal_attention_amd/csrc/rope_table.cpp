// Host-side RoPE cos/sin table builder.
//
// The page titled "手写内核实现6倍prefill加速" (§3.1) keeps cos(i*theta_k) and
// sin(i*theta_k) in position-indexed tables (length = max seq_len, ordered by
// theta_k, read as aligned pairs); the 2kiu.com retelling (§3.3, §4.2) builds
// the table offline at high precision and rounds once to fixed point.  Here the
// angle p*theta_k and its cos/sin are evaluated in fp64 on the host, then
// rounded once: to fp32 (cos, sin) pairs for the fp32 kernels and decode, to
// fp16 pairs for the bf16 prefill kernels (whose rotated Q' and K' are fp16
// anyway: half the table bytes per staged key), and to Q1.14 int16 (C, S)
// pairs for the fixed-point kernel.  Interleaving cos and sin of
// one pair lets a kernel fetch both with a single aligned load.

#include <cmath>
#include <cstdint>
#include <vector>

#include "internal.h"
#include "prefill_attn.h"

namespace {

bool table_args_ok(int max_seq, int head_dim, double rope_theta, const void* out) {
    return out != nullptr && max_seq > 0 && head_dim > 0 && (head_dim % 2) == 0 &&
           std::isfinite(rope_theta) && rope_theta > 0.0;
}

// theta_k = rope_theta^(-2k/head_dim), with the exponent formed as (-2k)/head_dim in fp64.
std::vector<double> inverse_frequencies(int head_dim, double rope_theta) {
    std::vector<double> inv(head_dim / 2);
    for (int k = 0; k < head_dim / 2; ++k)
        inv[k] = std::pow(rope_theta, (-2.0 * k) / head_dim);
    return inv;
}

// Fills either table (a null pointer is skipped) from one fp64 evaluation of
// each angle's cos and sin.
void fill_tables(int max_seq, int head_dim, double rope_theta, float* f32, int16_t* q14) {
    const int half = head_dim / 2;
    const std::vector<double> inv = inverse_frequencies(head_dim, rope_theta);
    for (int p = 0; p < max_seq; ++p) {
        const size_t row = static_cast<size_t>(p) * head_dim;
        for (int k = 0; k < half; ++k) {
            const double a = static_cast<double>(p) * inv[k];
            const double c = std::cos(a), s = std::sin(a);
            if (f32) {
                f32[row + 2 * k + 0] = static_cast<float>(c);
                f32[row + 2 * k + 1] = static_cast<float>(s);
            }
            if (q14) {
                // |cos|, |sin| <= 1, so the rounded value lies in [-16384, 16384]: fits int16.
                q14[row + 2 * k + 0] = static_cast<int16_t>(std::lround(c * 16384.0));
                q14[row + 2 * k + 1] = static_cast<int16_t>(std::lround(s * 16384.0));
            }
        }
    }
}

}  // namespace

namespace pa {
// The fp32 and Q1.14 tables from one pass (used by init).
int build_rope_tables(int max_seq, int head_dim, double rope_theta, float* f32, int16_t* q14) {
    if (!table_args_ok(max_seq, head_dim, rope_theta, f32) || !q14) return PA_EINVAL;
    fill_tables(max_seq, head_dim, rope_theta, f32, q14);
    return PA_OK;
}
}  // namespace pa

extern "C" int prefill_attn_rope_table_f32(int max_seq, int head_dim, double rope_theta, float* out) {
    if (!table_args_ok(max_seq, head_dim, rope_theta, out)) return PA_EINVAL;
    fill_tables(max_seq, head_dim, rope_theta, out, nullptr);
    return PA_OK;
}

extern "C" int prefill_attn_rope_table_q14(int max_seq, int head_dim, double rope_theta, int16_t* out) {
    if (!table_args_ok(max_seq, head_dim, rope_theta, out)) return PA_EINVAL;
    fill_tables(max_seq, head_dim, rope_theta, nullptr, out);
    return PA_OK;
}

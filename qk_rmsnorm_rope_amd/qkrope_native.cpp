// qkrope_native.cpp -- the two page signatures' calls marshalled in C++ onto the C ABI of
// include/qkrope.h (libqkrope.so), for callers that pay the host cost on every call:
//   table(...)  -> vLLM-Omni "vllm_omni.diffusion.layers.fused_qk_norm_rope", fused_qk_norm_rope
//   rope3d(...) -> FlashInfer "flashinfer.norm.fused_qk_rmsnorm_rope"
// Argument marshalling only, as the Python binding does it (same checks, same messages): shapes
// and strides from the tensors, outputs allocated with torch's allocator, the device's current
// stream, one C call. No arithmetic on the data happens here; every step runs in the library's
// HIP kernels. A status other than QKROPE_OK raises ValueError (invalid or unsupported
// arguments) or RuntimeError (device errors), each with the library's message.
#include <torch/extension.h>
#include <c10/hip/HIPStream.h>
#include <pybind11/stl.h>

#include <mutex>
#include <optional>
#include <string>

#include "qkrope.h"

namespace {

namespace py = pybind11;

constexpr int kMaxDevices = 64;
std::mutex g_mu;
qkrope_handle g_handles[kMaxDevices];

qkrope_handle handle_for(int dev)
{
    if (dev < 0 || dev >= kMaxDevices) throw py::value_error("device index out of range");
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_handles[dev]) {
        qkrope_handle h = nullptr;
        const int st = qkrope_create(dev, &h);
        if (st != QKROPE_OK)
            throw std::runtime_error(std::string("qkrope_create: ") + qkrope_status_str(st) + ": " +
                                     qkrope_last_error());
        g_handles[dev] = h;
    }
    return g_handles[dev];
}

void check_status(int st, const char *what)
{
    if (st == QKROPE_OK) return;
    const std::string msg = std::string(what) + ": " + qkrope_status_str(st) + ": " + qkrope_last_error();
    if (st == QKROPE_ERR_INVALID || st == QKROPE_ERR_UNSUPPORTED) throw py::value_error(msg);
    throw std::runtime_error(msg);
}

const char *dtype_name(at::ScalarType t)
{
    switch (t) {
    case at::kBFloat16: return "torch.bfloat16";
    case at::kHalf: return "torch.float16";
    case at::kFloat: return "torch.float32";
    case at::kFloat8_e4m3fn: return "torch.float8_e4m3fn";
    default: return "another dtype";
    }
}

int dtype_code(at::ScalarType t)
{
    switch (t) {
    case at::kBFloat16: return QKROPE_DTYPE_BF16;
    case at::kHalf: return QKROPE_DTYPE_F16;
    case at::kFloat: return QKROPE_DTYPE_F32;
    default: return -1;
    }
}

// Every given tensor must be a GPU tensor on the first input's device: the library reads and
// writes through the raw pointers.
void same_device(const at::Device &dev, const std::optional<at::Tensor> &t, const char *name)
{
    if (!t) return;
    if (!t->is_cuda() || t->device() != dev)
        throw py::value_error(std::string(name) + " must be a GPU tensor on " + dev.str() +
                              ", got " + t->device().str());
}

// A norm weight: contiguous, of `dtype`, holding at least the `need` elements the kernels read;
// a region that reads none may pass None.
void check_weight(const std::optional<at::Tensor> &w, int64_t need, at::ScalarType dtype,
                  const char *name)
{
    if (!w && need == 0) return;
    if (!w || w->scalar_type() != dtype || !w->is_contiguous() || w->numel() < need)
        throw py::value_error(std::string(name) + " must be a contiguous " + dtype_name(dtype) +
                              " tensor of at least " + std::to_string(need) + " elements");
}

// Token stride (elements) of a [T, H, D] (or [T, H*D]) view with contiguous heads and dims.
int64_t rows(const at::Tensor &t, int64_t heads, int64_t D, const char *name)
{
    bool ok;
    if (t.dim() == 3)
        ok = t.size(1) == heads && t.size(2) == D && (t.size(1) <= 1 || t.stride(1) == D) &&
             (t.size(2) <= 1 || t.stride(2) == 1);
    else if (t.dim() == 2)
        ok = t.size(1) == heads * D && (t.size(1) <= 1 || t.stride(1) == 1);
    else
        ok = false;
    if (!ok)
        throw py::value_error(std::string(name) +
                              " must be [tokens, heads, head_dim] with contiguous heads and dims");
    return t.size(0) > 1 ? t.stride(0) : heads * D;
}

void *ptr(const std::optional<at::Tensor> &t) { return t ? t->data_ptr() : nullptr; }

std::string i128_str(__int128 v)
{
    if (v >= INT64_MIN && v <= INT64_MAX) return std::to_string((int64_t)v);
    return std::to_string((double)v);
}

// An argument the C ABI takes as `int`: a larger value would reach it as its low 32 bits.
int c_int(int64_t v, const char *name)
{
    if (v < INT32_MIN || v > INT32_MAX)
        throw py::value_error(std::string(name) + " = " + std::to_string(v) +
                              " does not fit the C ABI's 32-bit int");
    return (int)v;
}

// fused_qk_norm_rope: per-head RMSNorm with [head_dim] weights, then RoPE from the packed
// [tokens, rotary_dim] = [cos | sin] table (its two halves are passed as the split tables).
py::tuple table(const at::Tensor &q, const at::Tensor &k, const std::optional<at::Tensor> &q_weight,
                const std::optional<at::Tensor> &k_weight, const at::Tensor &rope_table,
                double eps, std::optional<int64_t> head_dim, std::optional<int64_t> rotary_dim,
                bool interleaved)
{
    if (head_dim) c_int(*head_dim, "head_dim");
    if (rotary_dim) c_int(*rotary_dim, "rotary_dim");
    const int act = dtype_code(q.scalar_type());
    if ((act != QKROPE_DTYPE_BF16 && act != QKROPE_DTYPE_F16) || k.scalar_type() != q.scalar_type())
        throw py::value_error("q and k must both be bfloat16 or both float16");
    if (!q.is_cuda()) throw py::value_error("q must be a GPU tensor");
    if (!k.is_cuda()) throw py::value_error("k must be a GPU tensor");
    const int64_t D = head_dim ? *head_dim : q.size(-1);
    if (D <= 0) throw py::value_error("head_dim must be positive");
    const int64_t Hq = q.dim() == 3 ? q.size(1) : q.size(1) / D;
    const int64_t Hk = k.dim() == 3 ? k.size(1) : k.size(1) / D;
    const int64_t T = q.size(0);
    if (k.size(0) != T) throw py::value_error("q, k and outputs must have the same number of tokens");
    const int64_t R = rotary_dim ? *rotary_dim : rope_table.size(-1);
    const int tdt = dtype_code(rope_table.scalar_type());
    if (tdt != QKROPE_DTYPE_F32 && tdt != act)
        throw py::value_error("cos and sin tables must both be float32 or both the activation dtype");
    if (rope_table.dim() != 2 || rope_table.size(0) != T || rope_table.size(1) < R ||
        !rope_table.is_cuda() || (R > 0 && rope_table.size(1) > 1 && rope_table.stride(1) != 1))
        throw py::value_error("rope_table must be a GPU [tokens, >= rotary_dim] tensor whose "
                              "columns are contiguous (unit stride along the last dim)");
    const int64_t ts = T > 1 ? rope_table.stride(0) : rope_table.size(1);
    check_weight(q_weight, Hq > 0 ? D : 0, q.scalar_type(), "q_weight");
    check_weight(k_weight, Hk > 0 ? D : 0, q.scalar_type(), "k_weight");
    const at::Device dev = q.device();
    same_device(dev, k, "k");
    same_device(dev, rope_table, "rope_table");
    same_device(dev, q_weight, "q_weight");
    same_device(dev, k_weight, "k_weight");
    const int64_t qs = rows(q, Hq, D, "q"), ks = rows(k, Hk, D, "k");
    at::Tensor q_out = at::empty(q.sizes(), q.options());
    at::Tensor k_out = at::empty(k.sizes(), k.options());
    const int idx = dev.index();
    const auto *tab = static_cast<const uint8_t *>(rope_table.data_ptr());
    const void *sin = tab ? tab + (R / 2) * rope_table.element_size() : nullptr;
    const int st = qkrope_run_table_ex(
        handle_for(idx), q.data_ptr(), k.data_ptr(), ptr(q_weight), ptr(k_weight), tab, sin, tdt,
        act, act, 1.0, eps, T, c_int(Hq, "num_heads_q"), c_int(Hk, "num_heads_k"),
        c_int(D, "head_dim"), c_int(R, "rotary_dim"), interleaved ? 1 : 0,
        QKROPE_NORM_PER_HEAD, qs, ks, ts, ts, q_out.data_ptr(), k_out.data_ptr(),
        rows(q_out, Hq, D, "q_out"), rows(k_out, Hk, D, "k_out"),
        c10::hip::getCurrentHIPStream(idx).stream());
    check_status(st, "qkrope_run_table_ex");
    return py::make_tuple(q_out, k_out);
}

// fused_qk_rmsnorm_rope: across-heads RMSNorm, 3D RoPE, V copy, optional E4M3 outputs, into
// the given outputs or new ones shaped [B, S, H, D] (3D qkv) or [T, H, D] (2D qkv).
py::tuple rope3d(const at::Tensor &qkv, const std::optional<at::Tensor> &q_weight,
                 const std::optional<at::Tensor> &k_weight, int64_t ppf, int64_t pph, int64_t ppw,
                 int64_t cf, int64_t ch, int64_t cw, int64_t Hq, int64_t Hk, int64_t Hv,
                 int64_t D, double eps, double base, bool interleave, double factor, double low,
                 double high, double attention_factor, bool is_qk_norm, bool output_fp8,
                 double output_quant_scale, double v_quant_scale,
                 std::optional<at::Tensor> q_out, std::optional<at::Tensor> k_out,
                 std::optional<at::Tensor> v_out)
{
    const int ippf = c_int(ppf, "ppf"), ipph = c_int(pph, "pph"), ippw = c_int(ppw, "ppw");
    const int icf = c_int(cf, "num_frame_channels"), ich = c_int(ch, "num_height_channels"),
              icw = c_int(cw, "num_width_channels");
    const int iHq = c_int(Hq, "num_heads_q"), iHk = c_int(Hk, "num_heads_k"),
              iHv = c_int(Hv, "num_heads_v"), iD = c_int(D, "head_dim");
    // products of 32-bit values, formed in 128 bits (no overflow for any of them)
    const __int128 row128 = (__int128)(Hq + Hk + Hv) * D;
    const __int128 seq128 = (__int128)ppf * pph * ppw;
    if ((qkv.dim() != 2 && qkv.dim() != 3) || (__int128)qkv.size(-1) != row128)
        throw py::value_error("qkv must be [tokens, " + i128_str(row128) + "] or [batch, seq_len, " +
                              i128_str(row128) + "]");
    if (qkv.dim() == 3 && (__int128)qkv.size(1) != seq128)
        throw py::value_error("a [batch, seq_len, row] qkv needs seq_len == ppf*pph*ppw = " +
                              i128_str(seq128) + ", got " + std::to_string(qkv.size(1)));
    const int64_t row = qkv.size(-1);
    if (qkv.scalar_type() != at::kBFloat16 || !qkv.is_cuda() || !qkv.is_contiguous())
        throw py::value_error("qkv must be a contiguous bfloat16 GPU tensor");
    const int64_t T = row > 0 ? qkv.numel() / row : 0;
    const at::ScalarType odt = output_fp8 ? at::kFloat8_e4m3fn : at::kBFloat16;
    const at::Device dev = qkv.device();
    std::optional<at::Tensor> *outs[3] = {&q_out, &k_out, &v_out};
    const int64_t heads[3] = {Hq, Hk, Hv};
    const char *names[3] = {"q_out", "k_out", "v_out"};
    std::vector<int64_t> shape(qkv.sizes().begin(), qkv.sizes().end() - 1);
    shape.push_back(0);
    shape.push_back(D);
    for (int i = 0; i < 3; ++i) {
        std::optional<at::Tensor> &o = *outs[i];
        if (!o) {
            shape[shape.size() - 2] = heads[i];
            o = at::empty(shape, qkv.options().dtype(odt));
        } else if (o->scalar_type() != odt || !o->is_contiguous() || o->numel() != T * heads[i] * D ||
                   !o->is_cuda()) {
            throw py::value_error(std::string(names[i]) + " must be a contiguous " + dtype_name(odt) +
                                  " GPU tensor of " + std::to_string(T) + "x" +
                                  std::to_string(heads[i]) + "x" + std::to_string(D));
        }
    }
    if (is_qk_norm) {
        check_weight(q_weight, Hq * D, at::kBFloat16, "q_weight");
        check_weight(k_weight, Hk * D, at::kBFloat16, "k_weight");
    }
    same_device(dev, q_out, "q_out");
    same_device(dev, k_out, "k_out");
    same_device(dev, v_out, "v_out");
    if (is_qk_norm) {
        same_device(dev, q_weight, "q_weight");
        same_device(dev, k_weight, "k_weight");
    }
    const int idx = dev.index();
    const int st = qkrope_run_3d(
        handle_for(idx), qkv.data_ptr(), is_qk_norm ? ptr(q_weight) : nullptr,
        is_qk_norm ? ptr(k_weight) : nullptr, T, ippf, ipph, ippw, icf, ich, icw, iHq, iHk, iHv,
        iD, eps, base, interleave ? 1 : 0, factor, low,
        high, attention_factor, is_qk_norm ? 1 : 0, output_fp8 ? 1 : 0, output_quant_scale,
        v_quant_scale, q_out->data_ptr(), k_out->data_ptr(), v_out->data_ptr(),
        c10::hip::getCurrentHIPStream(idx).stream());
    check_status(st, "qkrope_run_3d");
    return py::make_tuple(*q_out, *k_out, *v_out);
}

}  // namespace

PYBIND11_MODULE(_qkrope_native, m)
{
    m.doc() = "C++ marshalling of the page signatures onto the qkrope C ABI";
    m.def("table", &table);
    m.def("rope3d", &rope3d);
}

"""Independent CPU cross-check of the oracle: explicit im2col followed by one matmul.

Follows the "Convolutions" tutorial page, section 5 ("How convolution becomes
GEMM") and its exercise A: the input of one image, taken channels-first as
(C_in, D, H, W), is unrolled into a matrix with one row per (c, kd, kh, kw)
and one column per output position; the weights are reshaped to
(C_out, C_in*KD*KH*KW) in the same row order; the convolution is the product
Weights @ im2col.  Everything is float64 numpy, built with array slicing (no
loop over output positions), so it shares neither code nor loop structure
with the oracle's direct loop nest.  Tiny shapes only: the unrolled matrix is
KD*KH*KW times the input.
"""
import numpy as np


def _extent(size, k, s, p):
    return (size + 2 * p - k) // s + 1


def im2col_matrix(x_chw, ksize, stride, pad):
    """(C, D, H, W) -> (C*KD*KH*KW, D_out*H_out*W_out), zero padding outside the input."""
    c, d, h, w = x_chw.shape
    kd, kh, kw = ksize
    sd, sh, sw = stride
    pd, ph, pw = pad
    od, oh, ow = _extent(d, kd, sd, pd), _extent(h, kh, sh, ph), _extent(w, kw, sw, pw)
    # Pad far enough on the high side that every strided slice below stays in range.
    hi = (max(0, (od - 1) * sd + kd - d - pd), max(0, (oh - 1) * sh + kh - h - ph),
          max(0, (ow - 1) * sw + kw - w - pw))
    xp = np.pad(x_chw, ((0, 0), (pd, hi[0]), (ph, hi[1]), (pw, hi[2])))
    cols = np.empty((c, kd, kh, kw, od * oh * ow), dtype=np.float64)
    for a in range(kd):
        for b in range(kh):
            for e in range(kw):
                patch = xp[:, a:a + (od - 1) * sd + 1:sd, b:b + (oh - 1) * sh + 1:sh,
                           e:e + (ow - 1) * sw + 1:sw]
                cols[:, a, b, e, :] = patch.reshape(c, -1)
    return cols.reshape(c * kd * kh * kw, od * oh * ow), (od, oh, ow)


def conv_im2col(x, w, stride, pad):
    """x: (N, D, H, W, C_in) float64; w: (C_out, KD, KH, KW, C_in).  Returns (N, Do, Ho, Wo, C_out)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    c_out = w.shape[0]
    wmat = np.transpose(w, (0, 4, 1, 2, 3)).reshape(c_out, -1)     # (C_out, C_in*KD*KH*KW)
    outs = []
    for img in x:
        cols, (od, oh, ow) = im2col_matrix(np.transpose(img, (3, 0, 1, 2)), w.shape[1:4],
                                           stride, pad)
        y = wmat @ cols                                               # (C_out, Do*Ho*Wo)
        outs.append(y.T.reshape(od, oh, ow, c_out))
    return np.stack(outs) if outs else np.zeros((0,), dtype=np.float64)

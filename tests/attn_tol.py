"""The per-element bar for comparing a binary32 implementation of attention on NVFP4
operands with the oracle (ScaleSearch summary page, ScaleSearchAttention, ネイティブ
NVFP4 実行: QK^T and PV with NVFP4 operands and FP32 accumulation).

The implementation under test forms every product exactly (the operands are
V[code] * s values), sums in FP32, computes p from binary32 scores and exp, and
keeps the online softmax over tiles of `tile` keys. Against the oracle (double
sums, p rounded once), its output differs through (u = 2^-24):

- the FP32 sum of P^ v into the accumulator, in steps of at most `tile` keys,
  tile after tile: each step rounds at most `tile` times at sizes up to
  |acc| + sum |P^ v| of the step, plus one rescale multiply per tile:
  (tile + 1) u rs + tile u mag, with rs = sum over tiles of |acc| as the tile
  starts and mag = sum |P^ v| (both in units of O, returned by the oracle);
- split keys: the merge of `units` states, sum_u w_u acc_u and sum_u w_u l_u in
  FP32: units u (us + |O|), us = sum_u |w_u acc_u|;
- rounded exponentials (each rescale factor, each merge weight): a relative
  error e on the weight of a group of keys moves O by at most e (mag + |O|);
  8 u each, for the tiles that may move the running max (nres), the merge and
  two spare;
- P coded against a running max other than the final one: binary32 scores put
  an error of up to dmax on each running max, and P's codes do not follow it
  (they are relative to the block's own max), so the weight of such keys moves
  by up to dmax: dmax mp, mp the magnitude sum of those keys (the tiles before
  the last possible rise of the max; every key of units other than the one
  holding the overall max);
- the softmax sum l: relative error dmax from p itself (binary32 scores and
  exp; the oracle's allowance) plus the FP32 sum along a key's chain: up to
  `tile` adds inside a tile, two per later tile, the merge and the output
  scaling: |O| (dmax + (2 ntiles + tile + 16 + units) u);
- P codes that round the other way (p near an E2M1 or E4M3 midpoint): the
  oracle's `bound`;
- bf16 output: |O| 2^-8.
"""
import numpy as np

U = 2.0 ** -24


def attention_tol(O, mag, bound, terms, tile: int = 32, out_bf16: bool = False):
    a = np.abs(O)
    col = lambda k: np.asarray(terms[k], np.float64)[..., None]
    nres, ntiles, dmax, units = col("nres"), col("ntiles"), col("dmax"), col("units")
    tol = ((tile + 1) * terms["rs"] + tile * mag) * U
    tol = tol + np.where(units > 1, units * (terms["us"] + a) * U, 0.0)
    tol = tol + (nres + 3) * 8 * U * (mag + a)
    tol = tol + dmax * terms["mp"]
    tol = tol + a * (dmax + (2 * ntiles + tile + 16 + units) * U)
    tol = tol + bound
    if out_bf16:
        tol = tol + a * 2.0 ** -8
    return tol
